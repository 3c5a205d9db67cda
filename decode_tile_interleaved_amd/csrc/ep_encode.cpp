// ep_encode.cpp -- host encoder: row normalization, E8 quantization, the
// conditional model, sampled resolution selection and interleaved rANS tiles.
//
// Method: "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at
// Arbitrary Bitrates" (arXiv abstract, mlsanity index page).  The pages give
// the steps, not their internals; the choices made here (RMS row scale, a
// 7-context model built on E8's coset bit and even-sum parity, 10-bit
// frequencies, 64 or 16 interleaved states per 512- or 1024-vector tile,
// start states bit-packed at their length, each pair of states sharing one
// word region read from both ends) define the stream that ep_decode.hip
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
static float row_scale(double rms, double a) { return (float)((rms * a) * 0.5); }

// quantizes vector k of row r (container src, C columns) at stored scale g;
// false if a coordinate leaves the stream's value range
static bool quantize(const void *src, int dtype, int64_t C, int64_t r, int64_t k, float g, int32_t *v) {
  if (g == 0.0f) {
    for (int j = 0; j < 8; ++j) v[j] = 0;
    return true;
  }
  double u[8];
  const double two_g = 2.0 * (double)g;
  for (int j = 0; j < 8; ++j) {
    int64_t c = 8 * k + j;
    double x = c < C ? widen(src, dtype, r * C + c) : 0.0;
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
// normalized frequency tables
// ---------------------------------------------------------------------------
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

static bool build_tables(const std::vector<uint64_t> &h, Tables &t) {
  for (int c = 0; c < kContexts; ++c) {
    int lo = kSymSpan, hi = -1;
    for (int i = 0; i < kSymSpan; ++i)
      if (h[(size_t)c * kSymSpan + i]) {
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
    if (!normalize(&h[(size_t)c * kSymSpan + lo], hi - lo + 1, t.freq[c])) return false;
    t.smin[c] = (int16_t)(lo - kSymBias);
    t.nsym[c] = (uint16_t)t.freq[c].size();
    t.cum[c].assign(t.freq[c].size() + 1, 0);
    for (size_t i = 0; i < t.freq[c].size(); ++i) t.cum[c][i + 1] = t.cum[c][i] + t.freq[c][i];
  }
  return true;
}

// ---------------------------------------------------------------------------
// the passes over the matrix on host threads
// ---------------------------------------------------------------------------
struct TileOut {
  std::vector<uint16_t> words;  // the tile as the stream stores it
  bool overflow = false;        // a pair's word count does not fit its count byte
};

class HostBackend final : public EncodeBackend {
 public:
  HostBackend(const void *src, const EncodeShape &S, int threads) : src_(src), S_(S), threads_(threads) {}

  int row_rms(std::vector<double> &rms, std::string &err) override {
    rms.assign((size_t)S_.R, 0.0);
    std::atomic<bool> bad{false};
    parallel_for(S_.R, threads_, [&](int64_t b, int64_t e) {
      for (int64_t r = b; r < e; ++r) {
        double acc = 0.0;
        for (int64_t c = 0; c < S_.C; ++c) {
          double x = widen(src_, S_.dtype, r * S_.C + c);
          if (!std::isfinite(x)) bad = true;
          acc += x * x;
        }
        rms[(size_t)r] = std::sqrt(acc / (double)S_.C);
      }
    });
    if (!bad) return 0;
    err = "input holds NaN or Inf";
    return EP_ERR_NONFINITE;
  }

  int histogram(const std::vector<float> &g, int64_t S, uint64_t seed, std::vector<uint64_t> &hist,
                std::string &) override {
    if (S >= S_.n_vec) return full_pass(g, hist);
    const int nt = std::max(1, std::min(threads_, 16));
    std::vector<std::vector<uint64_t>> part(nt, std::vector<uint64_t>((size_t)kContexts * kSymSpan, 0));
    std::atomic<bool> overflow{false};
    std::vector<std::thread> pool;
    for (int t = 0; t < nt; ++t)
      pool.emplace_back([&, t]() {
        int32_t v[8];
        for (int64_t k = t * S / nt; k < (t + 1) * S / nt; ++k) {
          int64_t vid = sample_vid(S_.n_vec, k, S, seed);
          int64_t r = vid / S_.vpr;
          if (!quantize(src_, S_.dtype, S_.C, r, vid % S_.vpr, g[(size_t)r], v)) {
            overflow = true;
            return;
          }
          Coded cd = model(v);
          for (int j = 0; j < 8; ++j) ++part[t][(size_t)cd.ctx[j] * kSymSpan + cd.sym[j] + kSymBias];
        }
      });
    for (auto &th : pool) th.join();
    if (overflow) return 1;
    hist = std::move(part[0]);
    for (int t = 1; t < nt; ++t)
      for (size_t i = 0; i < hist.size(); ++i) hist[i] += part[t][i];
    return 0;
  }

  int encode_tiles(const std::vector<float> &g, const Tables &tb, std::vector<uint32_t> &tile_first,
                   std::string &err) override {
    if (V_.empty() || Vg_ != g) {  // the lattice vectors of the last full pass, if it was at these scales
      std::vector<uint64_t> ignored;
      if (full_pass(g, ignored) != 0) {
        err = "a lattice coordinate left the stream's value range";
        return EP_ERR_ARG;
      }
    }
    const int64_t tiles = tile_count(layout_, S_.R, S_.vpr, tile_vecs_);
    tiles_.assign((size_t)tiles, TileOut{});
    parallel_for(tiles, std::max(1, threads_), [&](int64_t b, int64_t e) {
      for (int64_t t = b; t < e; ++t) encode_tile(tb, t, tiles_[(size_t)t]);
    });
    tile_first.resize((size_t)tiles + 1);
    uint64_t w = 0;
    for (int64_t t = 0; t < tiles; ++t) {
      tile_first[(size_t)t] = (uint32_t)w;
      w += tiles_[(size_t)t].words.size();
      if (w > 0xffffffffull) {
        err = "stream too large for 32-bit tile offsets";
        return EP_ERR_SHAPE;
      }
    }
    tile_first[(size_t)tiles] = (uint32_t)w;
    for (const TileOut &to : tiles_)
      if (to.overflow) return 1;
    return 0;
  }

  int copy_words(uint16_t *dst, std::string &) override {
    for (const TileOut &t : tiles_) {
      std::memcpy(dst, t.words.data(), 2 * t.words.size());
      dst += t.words.size();
    }
    return 0;
  }

  int copy_input(uint8_t *dst, std::string &) override {
    std::memcpy(dst, src_, (size_t)S_.R * (size_t)S_.C * elem_bytes(S_.dtype));
    return 0;
  }

 private:
  // every vector quantized at row scales g (kept for encode_tiles) and
  // counted; 1 if a coordinate leaves the value range
  int full_pass(const std::vector<float> &g, std::vector<uint64_t> &hist) {
    V_.assign((size_t)(S_.R * S_.C8), 0);
    Vg_.clear();
    const int nt = std::max(1, threads_);
    std::vector<std::vector<uint64_t>> part(nt, std::vector<uint64_t>((size_t)kContexts * kSymSpan, 0));
    std::atomic<bool> overflow{false};
    std::atomic<int64_t> next{0};
    auto worker = [&](int t) {
      for (;;) {
        int64_t r0 = next.fetch_add(16);
        if (r0 >= S_.R || overflow) break;
        for (int64_t r = r0; r < std::min(S_.R, r0 + 16); ++r)
          for (int64_t k = 0; k < S_.vpr; ++k) {
            int32_t *v = &V_[(size_t)(r * S_.C8 + 8 * k)];
            if (!quantize(src_, S_.dtype, S_.C, r, k, g[(size_t)r], v)) {
              overflow = true;
              return;
            }
            Coded cd = model(v);
            for (int j = 0; j < 8; ++j) ++part[t][(size_t)cd.ctx[j] * kSymSpan + cd.sym[j] + kSymBias];
          }
      }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < nt; ++t) pool.emplace_back(worker, t);
    worker(0);
    for (auto &th : pool) th.join();
    if (overflow) {
      V_.clear();
      return 1;
    }
    Vg_ = g;
    hist = std::move(part[0]);
    for (int t = 1; t < nt; ++t)
      for (size_t i = 0; i < hist.size(); ++i) hist[i] += part[t][i];
    return 0;
  }

  // one tile: interleaved rANS in reverse decode order from x = L, then the
  // tile as the stream stores it (pair counts, length codes, start bits,
  // pair regions)
  void encode_tile(const Tables &tb, int64_t tile, TileOut &out) const {
    // (frequency, cumulative) of every coordinate, vector-major; absent
    // vectors (past the matrix) are marked by frequency 0
    const int n = tile_vecs_;
    std::vector<uint32_t> fc((size_t)n * 8 * 2, 0u);
    for (int i = 0; i < n; ++i) {
      const int64_t vid = tile_vector(layout_, S_.R, S_.vpr, tile_vecs_, tile, i);
      if (vid < 0) continue;
      const int32_t *v = &V_[(size_t)((vid / S_.vpr) * S_.C8 + 8 * (vid % S_.vpr))];
      Coded cd = model(v);
      for (int j = 0; j < 8; ++j) {
        int c = cd.ctx[j], s = cd.sym[j] - tb.smin[c];
        fc[(size_t)(i * 8 + j) * 2] = tb.freq[c][s];
        fc[(size_t)(i * 8 + j) * 2 + 1] = tb.cum[c][s];
      }
    }
    const int S = states_;
    uint32_t x[kStatesPerTile];
    for (int q = 0; q < S; ++q) x[q] = kStateLow;
    std::vector<uint16_t> emitted;  // emission order (reverse of consumption)
    std::vector<uint8_t> who;       // state that emitted each word
    emitted.reserve((size_t)n * 3);
    who.reserve((size_t)n * 3);
    const int steps = tile_vecs_ / S;
    for (int s = steps - 1; s >= 0; --s)
      for (int j = 7; j >= 0; --j)
        for (int q = S - 1; q >= 0; --q) {
          int i = s * S + q;
          uint32_t f = fc[(size_t)(i * 8 + j) * 2], c = fc[(size_t)(i * 8 + j) * 2 + 1];
          if (f == 0) continue;  // no vector here
          uint32_t st = x[q];
          if ((uint64_t)st >= ((uint64_t)f << (kStateTop - kProbBits))) {
            emitted.push_back((uint16_t)st);
            who.push_back((uint8_t)q);
            st >>= 16;
          }
          x[q] = (st / f) * kProbTotal + st % f + c;
        }
    // per-state words in consumption order
    std::vector<std::vector<uint16_t>> lane((size_t)S);
    for (size_t k = emitted.size(); k-- > 0;) lane[who[k]].push_back(emitted[k]);
    std::vector<uint16_t> &w = out.words;
    w.clear();
    w.reserve(emitted.size() + (size_t)S + 8);
    out.overflow = false;
    for (int q = 0; q < S; q += 4) {  // pair counts, two pairs to a word
      const size_t lo = lane[q].size() + lane[q + 1].size(), hi = lane[q + 2].size() + lane[q + 3].size();
      out.overflow |= lo > 255 || hi > 255;
      w.push_back((uint16_t)((lo & 0xff) | (hi & 0xff) << 8));
    }
    int bits[kStatesPerTile];
    for (int q = 0; q < S; ++q) bits[q] = 32 - __builtin_clz(x[q]);  // in [12, 27]
    for (int q = 0; q < S; q += 4)  // length codes, four to a word
      w.push_back((uint16_t)((bits[q] - 12) | (bits[q + 1] - 12) << 4 | (bits[q + 2] - 12) << 8 |
                             (bits[q + 3] - 12) << 12));
    // start states below their leading bit, least significant bit first
    uint64_t acc = 0;
    int nacc = 0;
    for (int q = 0; q < S; ++q) {
      acc |= (uint64_t)(x[q] & ((1u << (bits[q] - 1)) - 1u)) << nacc;
      nacc += bits[q] - 1;
      while (nacc >= 16) {
        w.push_back((uint16_t)acc);
        acc >>= 16;
        nacc -= 16;
      }
    }
    if (nacc > 0) w.push_back((uint16_t)acc);
    for (int q = 0; q < S; q += 2) {  // region of states q, q + 1
      w.insert(w.end(), lane[q].begin(), lane[q].end());
      w.insert(w.end(), lane[q + 1].rbegin(), lane[q + 1].rend());
    }
  }

  const void *src_;
  EncodeShape S_;
  int threads_;
  std::vector<int32_t> V_;  // lattice vectors of the last full pass, rows of C8 coordinates
  std::vector<TileOut> tiles_;  // the last encode_tiles
  std::vector<float> Vg_;   // the row scales they were quantized at
};

// ---------------------------------------------------------------------------
// the encoder's control flow, on any backend
// ---------------------------------------------------------------------------
namespace {

thread_local int64_t g_encodes = 0;  // full encodes of the current compress call

struct Problem {
  EncodeShape S;
  EncodeBackend *be;
  std::vector<double> rms;
  int64_t sample = kSampleVecs;
  uint64_t seed = 0;
};

uint64_t metadata_bytes(const EncodeShape &S, int total_symbols) {
  return kHeaderBytes + align16(4 * kContexts + 2 * (uint64_t)total_symbols) + align16(4 * (uint64_t)S.R) +
         align16(4 * (uint64_t)(S.tiles + 1));
}

// the least a stream of this shape and geometry costs (every state coding
// nothing), bits per element
double floor_bpp(const EncodeShape &S) {
  return (kStateMinBits * (double)((int64_t)S.states * S.tiles) + 8.0 * (double)metadata_bytes(S, kContexts)) /
         ((double)S.R * (double)S.C);
}

std::vector<float> row_scales(const Problem &P, double a) {
  std::vector<float> g((size_t)P.S.R);
  for (int64_t r = 0; r < P.S.R; ++r) g[(size_t)r] = row_scale(P.rms[(size_t)r], a);
  return g;
}

// storage estimate (bits per element) at lattice scale a from the tables of
// S vectors (S >= n_vec: the whole matrix, no entropy coding): the symbols'
// information, 18.5 bits per state, the padding and the metadata; infinite
// if a coordinate leaves the value range
double estimate_bpp(const Problem &P, double a, int64_t S, std::string &err, int &status) {
  std::vector<uint64_t> hist;
  const int rc = P.be->histogram(row_scales(P, a), S, P.seed, hist, err);
  if (rc < 0) status = rc;
  if (rc != 0) return INFINITY;
  Tables tb;
  if (!build_tables(hist, tb)) return INFINITY;
  double info = 0.0;
  for (int c = 0; c < kContexts; ++c)
    for (int i = 0; i < tb.nsym[c]; ++i) {
      uint64_t n = hist[(size_t)c * kSymSpan + (tb.smin[c] + i) + kSymBias];
      if (n) info += (double)n * ((double)kProbBits - std::log2((double)tb.freq[c][i]));
    }
  const double scale = S >= P.S.n_vec ? 1.0 : (double)P.S.n_vec / (double)S;
  const double n_states = (double)((int64_t)P.S.states * P.S.tiles);
  const double bits = info * scale + kStateBits * n_states + kTilePadBits * (double)P.S.tiles + kWordsPadBits +
                      8.0 * (double)metadata_bytes(P.S, tb.total_symbols());
  return bits / ((double)P.S.R * (double)P.S.C);
}

// bisection on log2(a) over sampled estimates; returns the probed a whose
// estimate is closest to the target
double choose_scale(const Problem &P, double target, double *closest, std::string &err, int &status) {
  const int64_t S = std::min(P.S.n_vec, P.sample);
  const double la0 = 0.5 * std::log2(17.079468445347132) - target;  // high-rate guess sqrt(2 pi e) 2^-target
  double lo = la0 - 1.0, hi = la0 + 1.0;
  double best_la = la0, best_gap = INFINITY, best_e = INFINITY;
  auto probe = [&](double la) {
    double e = estimate_bpp(P, std::exp2(la), S, err, status);
    double gap = std::fabs(e - target);
    if (gap < best_gap) {
      best_gap = gap;
      best_la = la;
      best_e = e;
    }
    return e;
  };
  double e_lo = probe(lo);
  for (int k = 0; k < 30 && e_lo < target && status == 0; ++k) e_lo = probe(lo -= 2.0);
  double e_hi = probe(hi);
  for (int k = 0; k < 30 && e_hi > target && status == 0; ++k) e_hi = probe(hi += 2.0);
  for (int it = 0; it < 40 && status == 0; ++it) {
    double mid = 0.5 * (lo + hi);
    double e = probe(mid);
    if (std::fabs(e - target) <= 5e-4 * target) break;
    (e > target ? lo : hi) = mid;
  }
  *closest = best_e;
  return std::exp2(best_la);
}

// the full stream at resolution a
int encode_at(const Problem &P, double a, double target, Blob &blob, std::string &err) {
  ++g_encodes;
  const EncodeShape &S = P.S;
  const std::vector<float> g = row_scales(P, a);
  std::vector<uint64_t> hist;
  int rc = P.be->histogram(g, S.n_vec, 0, hist, err);
  if (rc < 0) return rc;
  if (rc == 1) return EP_WARN_RAW;
  Tables tb;
  // a context that needs more than 2^10 symbols cannot be coded: an encoding
  // failure, like values outside the stream's range (the sampled estimate may
  // have seen fewer symbols than the whole matrix holds)
  if (!build_tables(hist, tb)) return EP_WARN_RAW;
  std::vector<uint32_t> tile_first;
  rc = P.be->encode_tiles(g, tb, tile_first, err);
  if (rc < 0) return rc;
  if (rc == 1) return EP_WARN_RAW;  // a count byte cannot hold a pair's words: an encoding failure
  const uint64_t n_words = tile_first.back();
  const int nsum = tb.total_symbols();
  const uint64_t o_tab = kHeaderBytes;
  const uint64_t o_sc = o_tab + align16(4 * kContexts + 2 * (uint64_t)nsum);
  const uint64_t o_to = o_sc + align16(4 * (uint64_t)S.R);
  const uint64_t o_w = o_to + align16(4 * (uint64_t)(S.tiles + 1));
  const uint64_t total = o_w + align16(2 * n_words);
  if (!blob.alloc(total)) {
    err = "host allocation failed";
    return EP_ERR_NOMEM;
  }
  uint8_t *b = blob.data();
  std::memset(b, 0, o_w);                                           // every section before the words, with its padding
  std::memset(b + o_w + 2 * n_words, 0, total - o_w - 2 * n_words);  // the words' padding
  wr<uint32_t>(b + hdr::magic, kMagic);
  wr<uint16_t>(b + hdr::version, kVersion);
  wr<uint16_t>(b + hdr::header_bytes, (uint16_t)kHeaderBytes);
  b[hdr::method] = kLattice;
  b[hdr::dtype] = (uint8_t)S.dtype;
  b[hdr::prob_bits] = kProbBits;
  b[hdr::contexts] = kContexts;
  wr<uint32_t>(b + hdr::tile_vecs, (uint32_t)S.tile_vecs);
  wr<uint32_t>(b + hdr::states, (uint32_t)S.states);
  wr<uint32_t>(b + hdr::tiles, (uint32_t)S.tiles);
  wr<uint64_t>(b + hdr::rows, (uint64_t)S.R);
  wr<uint64_t>(b + hdr::cols, (uint64_t)S.C);
  wr<uint64_t>(b + hdr::cols8, (uint64_t)S.C8);
  wr<double>(b + hdr::scale_a, a);
  wr<double>(b + hdr::target, target);
  wr<uint64_t>(b + hdr::off_tables, o_tab);
  wr<uint64_t>(b + hdr::off_scales, o_sc);
  wr<uint64_t>(b + hdr::off_states, 0);
  wr<uint64_t>(b + hdr::off_tile_offsets, o_to);
  wr<uint64_t>(b + hdr::off_words, o_w);
  wr<uint64_t>(b + hdr::n_words, n_words);
  wr<uint64_t>(b + hdr::total, total);
  b[hdr::layout] = (uint8_t)S.layout;
  uint8_t *p = b + o_tab + 4 * kContexts;
  for (int c = 0; c < kContexts; ++c) {
    wr<int16_t>(b + o_tab + 4 * c, tb.smin[c]);
    wr<uint16_t>(b + o_tab + 4 * c + 2, tb.nsym[c]);
    for (uint32_t f : tb.freq[c]) {
      wr<uint16_t>(p, (uint16_t)f);
      p += 2;
    }
  }
  std::memcpy(b + o_sc, g.data(), 4 * (size_t)S.R);
  std::memcpy(b + o_to, tile_first.data(), 4 * tile_first.size());
  return P.be->copy_words(reinterpret_cast<uint16_t *>(b + o_w), err);
}

int raw_stream(const Problem &P, double target, Blob &blob, std::string &err) {
  const EncodeShape &S = P.S;
  const uint64_t payload = (uint64_t)S.R * (uint64_t)S.C * elem_bytes(S.dtype);
  if (!blob.alloc(kHeaderBytes + align16(payload))) {
    err = "host allocation failed";
    return EP_ERR_NOMEM;
  }
  uint8_t *b = blob.data();
  std::memset(b, 0, kHeaderBytes);
  std::memset(b + kHeaderBytes + payload, 0, blob.size() - kHeaderBytes - payload);
  wr<uint32_t>(b + hdr::magic, kMagic);
  wr<uint16_t>(b + hdr::version, kVersion);
  wr<uint16_t>(b + hdr::header_bytes, (uint16_t)kHeaderBytes);
  b[hdr::method] = kRaw;
  b[hdr::dtype] = (uint8_t)S.dtype;
  wr<uint64_t>(b + hdr::rows, (uint64_t)S.R);
  wr<uint64_t>(b + hdr::cols, (uint64_t)S.C);
  wr<uint64_t>(b + hdr::cols8, (uint64_t)S.C);
  wr<double>(b + hdr::target, target);
  wr<uint64_t>(b + hdr::off_words, kHeaderBytes);
  wr<uint64_t>(b + hdr::total, (uint64_t)blob.size());
  return P.be->copy_input(b + kHeaderBytes, err);
}

}  // namespace

int64_t last_encode_count() { return g_encodes; }

bool make_shape(int dtype, int64_t rows, int64_t cols, EncodeShape &S, int &status, std::string &err) {
  if (dtype < 0 || dtype > 3) {
    err = "unknown container dtype";
    status = EP_ERR_ARG;
    return false;
  }
  if (rows <= 0 || cols <= 0) {
    err = "input must be a non-empty 2-D matrix";
    status = EP_ERR_SHAPE;
    return false;
  }
  if (rows >= (int64_t(1) << 31) || cols >= (int64_t(1) << 31)) {
    err = "matrix too large for one stream";
    status = EP_ERR_SHAPE;
    return false;
  }
  S.dtype = dtype;
  S.R = rows;
  S.C = cols;
  S.C8 = (cols + 7) / 8 * 8;
  S.vpr = S.C8 / 8;
  S.n_vec = rows * S.vpr;
  if (S.n_vec >= (int64_t(1) << 31)) {
    err = "matrix too large for one stream";
    status = EP_ERR_SHAPE;
    return false;
  }
  S.set_tiles(kStatesPerTile, S.n_vec < kSmallMatrixVecs ? kTileVecsSmall : kTileVecsLarge);
  return true;
}

int compress_with(EncodeBackend &be, const EncodeShape &shape, double target, const EncodeOptions &opt,
                  Blob &blob, std::string &err) {
  g_encodes = 0;
  if ((opt.n_states != 0 && opt.n_states != kStatesLow && opt.n_states != kStatesPerTile) ||
      (opt.tile_vecs != 0 && opt.tile_vecs != kTileVecsSmall && opt.tile_vecs != kTileVecsLarge) ||
      opt.sample_vecs < 0 || !(opt.fixed_a >= 0.0) || std::isinf(opt.fixed_a) ||
      (opt.layout != kLayoutRows && opt.layout != kLayoutBlocks)) {
    err = "invalid ep_options";
    return EP_ERR_ARG;
  }
  EncodeOptions o = opt;
  if (o.layout == kLayoutBlocks) {
    // the blocks layout feeds the fused linear's BF16 matrix multiply
    if (shape.dtype != EP_BF16 || (o.n_states != 0 && o.n_states != kStatesPerTile) ||
        (o.tile_vecs != 0 && o.tile_vecs != kTileVecsSmall)) {
      err = "the blocks layout takes BF16 matrices with 64-state, 512-vector tiles";
      return EP_ERR_ARG;
    }
    if (shape.C % 8 != 0) {
      err = "the blocks layout needs cols % 8 == 0";
      return EP_ERR_SHAPE;
    }
    o.n_states = kStatesPerTile;
    o.tile_vecs = kTileVecsSmall;
  }
  Problem P{shape, &be, {}, o.sample_vecs ? o.sample_vecs : kSampleVecs, o.seed};
  EncodeShape &S = P.S;
  S.layout = o.layout;
  const bool chosen = !(o.fixed_a > 0.0);
  // Tile geometry.  64 states per tile, or 16 when a target-selected
  // stream's target is less than 4x the least a 64-state stream costs (64
  // would spend over a quarter of the bits on their overhead).  64-state
  // tiles hold 512 vectors in matrices of fewer than 2^22 vectors (twice the
  // states decoding in parallel), else 1024; 16-state tiles hold 512, or
  // 1024 when the target lies below 1.1x the least 512 allow.
  const int tv64 = o.tile_vecs ? o.tile_vecs : (S.n_vec < kSmallMatrixVecs ? kTileVecsSmall : kTileVecsLarge);
  int states = o.n_states;
  if (!states) {
    S.set_tiles(kStatesPerTile, tv64);
    states = (chosen && target < 4.0 * floor_bpp(S)) ? kStatesLow : kStatesPerTile;
  }
  int tile_vecs = o.tile_vecs;
  if (!tile_vecs) {
    if (states == kStatesPerTile) {
      tile_vecs = tv64;
    } else {
      S.set_tiles(kStatesLow, kTileVecsSmall);
      tile_vecs = (chosen && target < 1.1 * floor_bpp(S)) ? kTileVecsLarge : kTileVecsSmall;
    }
  }
  S.set_tiles(states, tile_vecs);
  be.set_geometry(states, tile_vecs, S.layout);
  // finiteness and row RMS (sequential sum per row)
  if (const int rc = be.row_rms(P.rms, err); rc != 0) return rc;
  const bool eight_bit = elem_bytes(S.dtype) == 1;
  if (!std::isfinite(target) || target < 0.001 || (!eight_bit && target > 11.0) || (eight_bit && target >= 8.0)) {
    err = "target_bpp outside the supported range for this container";
    return EP_ERR_TARGET;
  }
  double a = o.fixed_a;
  if (chosen) {
    const double fl = floor_bpp(S);
    if (target < 1.02 * fl) {
      err = "target_bpp below this stream's fixed per-tile overhead (" + std::to_string(fl) + " bpp)";
      return EP_ERR_TARGET;
    }
    int status = 0;
    double closest;
    a = choose_scale(P, target, &closest, err, status);
    if (status < 0) return status;
    if (!(std::fabs(closest - target) <= 0.02 * target)) {
      const int rc = raw_stream(P, target, blob, err);
      if (rc < 0) return rc;
      err = "no lattice resolution reaches the target; stored the raw container";
      return EP_WARN_RAW;
    }
    // The sample misses rare symbols that the full tables must still give a
    // frequency of at least 1.  One histogram of the whole matrix at the chosen
    // scale (no entropy coding) measures that bias; beyond 0.5% the sampled
    // bisection runs again toward the target minus the bias.  The bias changes
    // with the scale, so this repeats (at most three bisections) until the
    // whole-matrix estimate is within 0.5% of the target.
    double full = estimate_bpp(P, a, S.n_vec, err, status);
    if (status < 0) return status;
    if (std::isfinite(full) && !(std::fabs(full - target) <= 0.005 * target)) {
      double est = closest;
      for (int it = 0; it < 3; ++it) {
        a = choose_scale(P, target - (full - est), &est, err, status);
        if (status < 0) return status;
        if (it == 2) break;
        full = estimate_bpp(P, a, S.n_vec, err, status);
        if (status < 0) return status;
        if (!std::isfinite(full) || std::fabs(full - target) <= 0.005 * target) break;
      }
    }
  }
  // the one full encode
  int rc = encode_at(P, a, target, blob, err);
  if (rc < 0) return rc;
  const uint64_t raw_total = kHeaderBytes + align16((uint64_t)S.R * (uint64_t)S.C * elem_bytes(S.dtype));
  if (rc == EP_OK && chosen && blob.size() >= raw_total) rc = EP_WARN_RAW;
  if (rc == EP_WARN_RAW) {
    const int rr = raw_stream(P, target, blob, err);
    if (rr < 0) return rr;
    err = "lattice coding failed (values out of range, a context beyond 2^10 symbols, a pair's words beyond its "
          "count byte, or no gain); stored the raw container";
  }
  return rc;
}

int compress(const void *src, int dtype, int64_t rows, int64_t cols, double target, const EncodeOptions &opt,
             int threads, Blob &blob, std::string &err) {
  EncodeShape S;
  int status = 0;
  if (!make_shape(dtype, rows, cols, S, status, err)) return status;
  if (!src) {
    err = "null input";
    return EP_ERR_ARG;
  }
  HostBackend be(src, S, threads > 0 ? threads : (int)std::max(1u, std::thread::hardware_concurrency()));
  return compress_with(be, S, target, opt, blob, err);
}

}  // namespace ep
