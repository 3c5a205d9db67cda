/*
 * oracle.c -- plain, slow CPU oracle for lattice-rANS weight compression.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or constant generator with the product library under
 * decode_tile_interleaved_amd/csrc; the two meet only through byte streams.
 *
 * What it computes follows "EntroPack: Fast and Accurate Entropy-Coded Weight
 * Compression at Arbitrary Bitrates" (arXiv abstract, mlsanity index page):
 * row-normalized E8 lattice quantization, a conditional probability model of
 * lattice coordinates, resolution selection from sampled storage estimates,
 * and entropy coding in independently decodable tiles.  The bpp definition
 * and input rules come from the EntroPack API reference page
 * (CompressedTensor.actual_bpp; compress input requirements).  Every step the
 * pages leave open is a stated reading; all arithmetic is scalar C in f64
 * (f32 only where the stored stream fixes f32: the per-row scale and the
 * reconstruction product).
 *
 * Parity pins for each function are listed in the oracle package docstring.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* status codes (numerically identical to the product ABI; defined here on
 * purpose so that the oracle includes nothing from the product) */
#define OR_OK 0
#define OR_WARN_RAW 1
#define OR_ERR_ARG (-1)
#define OR_ERR_SHAPE (-2)
#define OR_ERR_NONFINITE (-3)
#define OR_ERR_TARGET (-4)
#define OR_ERR_FORMAT (-5)
#define OR_ERR_NOMEM (-7)

/* container dtypes */
#define OR_BF16 0
#define OR_FP16 1
#define OR_FP8 2
#define OR_INT8 3

#define OR_NCTX 7
#define OR_HDR 128
#define OR_MAGIC 0x314B5045u /* "EPK1" little-endian */
#define OR_VERSION 2
#define OR_STATES_DEFAULT 64 /* rANS states per tile */
#define OR_STATES_LOW 16     /* per tile when the target is below the overhead of 64 */
#define OR_STATE_L 2048u     /* rANS lower state bound L = 2^11; states lie in [L, 2^27); words are 16 bits */
#define OR_STATE_TOP 27      /* log2(L) + 16: the encoder emits a word while x >= f * 2^(27 - prob_bits) */
/*
 * Stream bits a state costs beyond the information of its symbols, as the
 * rate estimate counts them.  A tile stores per state half a pair-count byte
 * and a 4-bit length code (8 bits), and the start state x_f at its bit length
 * W less its implicit leading one: W - 1 = floor(log2 x_f) bits.  The symbols'
 * information equals the words plus log2(x_f / L), so the state's own cost is
 * 8 + 11 + floor(log2 x_f) - log2 x_f, on average 18.5 bits; a state that
 * codes nothing costs 19.
 */
#define OR_STATE_BITS 18.5
#define OR_STATE_MIN_BITS 19.0
/* the start bits of a tile end on a whole word (7.5 bits of padding on
 * average), and the word section ends on 16 bytes (60 bits on average) */
#define OR_TILE_PAD_BITS 7.5
#define OR_WORDS_PAD_BITS 60.0
/* matrices of fewer E8 vectors than this get 512-vector tiles when they have
 * 64 states per tile (twice the tiles, so twice the parallel rANS states),
 * larger ones 1024-vector tiles */
#define OR_SMALL_MATRIX_VECS 4194304
/* stride sample of the rate estimate, vectors */
#define OR_SAMPLE_VECS 65536

static int esize_of(int dt) { return (dt == OR_BF16 || dt == OR_FP16) ? 2 : 1; }

/* ------------------------------------------------------------------------ */
/* little-endian byte access                                                 */
/* ------------------------------------------------------------------------ */
static void put_u16(uint8_t *p, uint32_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint32_t v) { for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static void put_u64(uint8_t *p, uint64_t v) { for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i)); }
static void put_f64(uint8_t *p, double d) { uint64_t u; memcpy(&u, &d, 8); put_u64(p, u); }
static void put_f32(uint8_t *p, float f) { uint32_t u; memcpy(&u, &f, 4); put_u32(p, u); }
static uint32_t get_u16(const uint8_t *p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }
static uint32_t get_u32(const uint8_t *p) {
  uint32_t v = 0;
  for (int i = 0; i < 4; i++) v |= (uint32_t)p[i] << (8 * i);
  return v;
}
static uint64_t get_u64(const uint8_t *p) {
  uint64_t v = 0;
  for (int i = 0; i < 8; i++) v |= (uint64_t)p[i] << (8 * i);
  return v;
}
static double get_f64(const uint8_t *p) { uint64_t u = get_u64(p); double d; memcpy(&d, &u, 8); return d; }
static float get_f32(const uint8_t *p) { uint32_t u = get_u32(p); float f; memcpy(&f, &u, 4); return f; }
static uint64_t pad16(uint64_t n) { return (n + 15) & ~(uint64_t)15; }

/* ------------------------------------------------------------------------ */
/* E8 nearest point: Conway & Sloane, fast quantizing for D_n and E8.        */
/* E8 = D8 U (D8 + 1/2), D8 = integer vectors with even sum.                 */
/* ------------------------------------------------------------------------ */
static void nearest_d8(const double *u, double *f) {
  double s = 0.0;
  for (int i = 0; i < 8; i++) {
    f[i] = nearbyint(u[i]); /* round half to even (default rounding mode) */
    s += f[i];
  }
  if (fmod(s, 2.0) != 0.0) {
    /* odd sum: move the coordinate with the largest rounding error one step
     * toward its input; the first such coordinate wins a tie */
    int w = 0;
    double wd = -1.0;
    for (int i = 0; i < 8; i++) {
      double d = fabs(u[i] - f[i]);
      if (d > wd) { wd = d; w = i; }
    }
    if (u[w] > f[w]) f[w] += 1.0;
    else if (u[w] < f[w]) f[w] -= 1.0;
    else f[w] += 1.0;
  }
}

/* v = 2 * (nearest E8 point to u); the D8 candidate wins an exact tie. */
int or_e8_nearest(const double *u, int32_t *v) {
  double a[8], b[8], h[8];
  nearest_d8(u, a);
  for (int i = 0; i < 8; i++) h[i] = u[i] - 0.5;
  nearest_d8(h, b);
  for (int i = 0; i < 8; i++) b[i] += 0.5;
  double da = 0.0, db = 0.0;
  for (int i = 0; i < 8; i++) {
    double ea = u[i] - a[i], eb = u[i] - b[i];
    da += ea * ea;
    db += eb * eb;
  }
  const double *y = (db < da) ? b : a;
  for (int i = 0; i < 8; i++) v[i] = (int32_t)(2.0 * y[i]);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Row normalization and per-row stored scale.                               */
/* s_r = RMS of row r (f64);  g_r = f32(s_r * a / 2);  u = x / (2 g_r).      */
/* A zero g_r codes the whole row as the lattice origin.                     */
/* ------------------------------------------------------------------------ */
static double row_rms(const double *row, int64_t C) {
  double acc = 0.0;
  for (int64_t c = 0; c < C; c++) acc += row[c] * row[c];
  return sqrt(acc / (double)C);
}

static float stored_scale(double s, double a) { return (float)((s * a) * 0.5); }

/* the 8 padded coordinates of vector k of row r, normalized by g */
static void normalized_vector(const double *row, int64_t C, int64_t k, float g, double *u) {
  for (int j = 0; j < 8; j++) {
    int64_t c = 8 * k + j;
    double x = (c < C) ? row[c] : 0.0;
    u[j] = x / (2.0 * (double)g);
  }
}

static void quantize_vector(const double *row, int64_t C, int64_t k, float g, int32_t *v) {
  if (g == 0.0f) {
    for (int j = 0; j < 8; j++) v[j] = 0;
    return;
  }
  double u[8];
  normalized_vector(row, C, k, g, u);
  or_e8_nearest(u, v);
}

/* ------------------------------------------------------------------------ */
/* Conditional model of the lattice coordinates (7 contexts).                */
/* coordinate 0: symbol v0 in context F (0); b = v0 & 1 is the coset bit.    */
/* coordinates 1..6: z = (v - b)/2 in context C_b (1 + b).                   */
/* coordinate 7: p = (z0 + .. + z6) & 1; since the z sum is even, z7 = p     */
/* (mod 2) and m = (z7 - p)/2 is coded in context E_{b,p} (3 + 2b + p).      */
/* ------------------------------------------------------------------------ */
static void vector_symbols(const int32_t *v, int *ctx, int32_t *sym) {
  int32_t b = v[0] & 1;
  int32_t zs = (v[0] - b) / 2;
  ctx[0] = 0;
  sym[0] = v[0];
  for (int j = 1; j < 7; j++) {
    int32_t z = (v[j] - b) / 2;
    ctx[j] = 1 + b;
    sym[j] = z;
    zs += z;
  }
  int32_t p = zs & 1;
  int32_t z7 = (v[7] - b) / 2;
  ctx[7] = 3 + 2 * b + p;
  sym[7] = (z7 - p) / 2;
}

/* inverse of the model for one coordinate, given b and p */
static int32_t symbol_value(int ctx, int32_t s, int32_t b, int32_t p) {
  if (ctx == 0) return s;
  if (ctx <= 2) return 2 * s + b;
  return 4 * s + 2 * p + b;
}

/* lattice coordinates v must fit the stream's signed value field */
static int value_bits(int prob_bits) { return 32 - 2 * prob_bits; }
static int value_in_range(int32_t v, int prob_bits) {
  int vb = value_bits(prob_bits);
  int32_t lo = -(1 << (vb - 1)), hi = (1 << (vb - 1)) - 1;
  return v >= lo && v <= hi;
}

/* ------------------------------------------------------------------------ */
/* Histograms and frequency normalization to M = 2^prob_bits.                */
/* ------------------------------------------------------------------------ */
#define OR_SYM_OFF 4096  /* histogram index = symbol + OR_SYM_OFF */
#define OR_SYM_SPAN 8192

typedef struct {
  uint64_t cnt[OR_NCTX][OR_SYM_SPAN];
} or_hist;

typedef struct {
  int32_t smin[OR_NCTX];
  int nsym[OR_NCTX];
  uint32_t *freq[OR_NCTX]; /* nsym entries each */
  uint32_t *cum[OR_NCTX];  /* nsym + 1 entries */
} or_tables;

static void tables_free(or_tables *t) {
  for (int c = 0; c < OR_NCTX; c++) {
    free(t->freq[c]);
    free(t->cum[c]);
    t->freq[c] = t->cum[c] = NULL;
  }
}

/*
 * f_s = 0 if c_s = 0, else max(1, floor((c_s*M + floor(N/2)) / N)).
 * d = M - sum f: d > 0 goes to the most frequent symbol (lowest index on a
 * tie); while d < 0 the symbol with the largest f > 1 (lowest index on a
 * tie) gives up one.  A context with a single used symbol gets f = M - 1 and
 * a never-used companion symbol (the next index) gets f = 1, so every
 * frequency fits in prob_bits bits.
 */
static int normalize_counts(const uint64_t *cnt, int nsym, int prob_bits, uint32_t *f, int *nsym_out) {
  uint64_t M = (uint64_t)1 << prob_bits;
  uint64_t N = 0;
  int used = 0;
  for (int s = 0; s < nsym; s++) {
    N += cnt[s];
    if (cnt[s]) used++;
  }
  *nsym_out = nsym;
  if (N == 0) return OR_OK;
  if (used == 1) {
    /* nsym is 1 here because the alphabet spans only used symbols */
    f[0] = (uint32_t)(M - 1);
    f[1] = 1;
    *nsym_out = 2;
    return OR_OK;
  }
  if ((uint64_t)used > M) return OR_ERR_TARGET;
  int64_t sum = 0;
  for (int s = 0; s < nsym; s++) {
    if (cnt[s] == 0) f[s] = 0;
    else {
      uint64_t q = (cnt[s] * M + N / 2) / N;
      f[s] = (uint32_t)(q < 1 ? 1 : q);
    }
    sum += f[s];
  }
  int64_t d = (int64_t)M - sum;
  if (d > 0) {
    int w = 0;
    for (int s = 1; s < nsym; s++)
      if (cnt[s] > cnt[w]) w = s;
    f[w] += (uint32_t)d;
  }
  while (d < 0) {
    int w = -1;
    for (int s = 0; s < nsym; s++)
      if (f[s] > 1 && (w < 0 || f[s] > f[w])) w = s;
    if (w < 0) return OR_ERR_TARGET;
    f[w] -= 1;
    d += 1;
  }
  return OR_OK;
}

/* alphabet = [min used symbol, max used symbol] per context */
static int tables_from_hist(const or_hist *h, int prob_bits, or_tables *t) {
  memset(t, 0, sizeof(*t));
  for (int c = 0; c < OR_NCTX; c++) {
    int lo = -1, hi = -1;
    for (int i = 0; i < OR_SYM_SPAN; i++)
      if (h->cnt[c][i]) {
        if (lo < 0) lo = i;
        hi = i;
      }
    if (lo < 0) {
      t->smin[c] = 0;
      t->nsym[c] = 0;
      t->freq[c] = (uint32_t *)calloc(2, sizeof(uint32_t));
      t->cum[c] = (uint32_t *)calloc(3, sizeof(uint32_t));
      if (!t->freq[c] || !t->cum[c]) return OR_ERR_NOMEM;
      continue;
    }
    int n = hi - lo + 1;
    t->smin[c] = lo - OR_SYM_OFF;
    t->freq[c] = (uint32_t *)calloc((size_t)n + 1, sizeof(uint32_t));
    t->cum[c] = (uint32_t *)calloc((size_t)n + 2, sizeof(uint32_t));
    if (!t->freq[c] || !t->cum[c]) return OR_ERR_NOMEM;
    int rc = normalize_counts(&h->cnt[c][lo], n, prob_bits, t->freq[c], &t->nsym[c]);
    if (rc) return rc;
    t->cum[c][0] = 0;
    for (int s = 0; s < t->nsym[c]; s++) t->cum[c][s + 1] = t->cum[c][s] + t->freq[c][s];
  }
  return OR_OK;
}

static int tables_total_nsym(const or_tables *t) {
  int n = 0;
  for (int c = 0; c < OR_NCTX; c++) n += t->nsym[c];
  return n;
}

/* ------------------------------------------------------------------------ */
/* Problem geometry                                                          */
/* ------------------------------------------------------------------------ */
typedef struct {
  int64_t R, C, Cp;    /* rows, columns, columns padded to a multiple of 8 */
  int64_t vpr;         /* vectors per row */
  int64_t n_vec;
  int64_t tile_vecs;   /* E8 vectors per tile: a multiple of S */
  int64_t S;           /* rANS states per tile (16 or 64) */
  int64_t T;           /* tiles */
  int prob_bits;
  int layout;          /* OR_LAYOUT_ROWS or OR_LAYOUT_BLOCKS */
  int64_t KB;          /* blocks layout: blocks per block row (ceil(vpr / 8)) */
} or_geom;

/*
 * Tile layouts.  The pages ask for independently decodable tiles and leave
 * their shape open.
 *   OR_LAYOUT_ROWS:   tile t holds vectors t*tile_vecs .. in row-major vector
 *                     order (the last tile may be partial).
 *   OR_LAYOUT_BLOCKS: the weight block of rows 64*nb .. 64*nb + 63 and vector
 *                     columns 8*kb .. 8*kb + 7 (64 columns) is tile
 *                     t = nb*KB + kb; its local vector i sits at row
 *                     64*nb + i/8, vector column 8*kb + i%8, and is absent
 *                     (coded by nobody) where that lies outside the matrix.
 *                     A matrix product reads W one such block at a time, so a
 *                     GPU can decode each block straight into the operand of a
 *                     matrix multiply (API reference, "CompressedLinear":
 *                     reconstructed weights feed every forward call).  512
 *                     vectors and 64 states per tile.
 */
#define OR_LAYOUT_ROWS 0
#define OR_LAYOUT_BLOCKS 1
#define OR_BLOCK_ROWS 64
#define OR_BLOCK_VECS 8

static void geom_init(or_geom *g, int64_t R, int64_t C, int64_t S, int64_t tile_vecs, int prob_bits, int layout) {
  g->R = R;
  g->C = C;
  g->Cp = (C + 7) / 8 * 8;
  g->vpr = g->Cp / 8;
  g->n_vec = R * g->vpr;
  g->tile_vecs = tile_vecs;
  g->S = S;
  g->prob_bits = prob_bits;
  g->layout = layout;
  g->KB = (g->vpr + OR_BLOCK_VECS - 1) / OR_BLOCK_VECS;
  if (layout == OR_LAYOUT_BLOCKS)
    g->T = (R + OR_BLOCK_ROWS - 1) / OR_BLOCK_ROWS * g->KB;
  else
    g->T = (g->n_vec + g->tile_vecs - 1) / g->tile_vecs;
}

/* the global vector index (row * vpr + vector column) of local vector i of
 * tile t, or -1 where the tile has no such vector */
static int64_t tile_vector(const or_geom *g, int64_t t, int64_t i) {
  if (g->layout == OR_LAYOUT_BLOCKS) {
    int64_t r = (t / g->KB) * OR_BLOCK_ROWS + i / OR_BLOCK_VECS;
    int64_t k = (t % g->KB) * OR_BLOCK_VECS + i % OR_BLOCK_VECS;
    if (r >= g->R || k >= g->vpr) return -1;
    return r * g->vpr + k;
  }
  int64_t vid = t * g->tile_vecs + i;
  return vid < g->n_vec ? vid : -1;
}

/* bytes of everything except the word section, with section padding */
static uint64_t meta_bytes(const or_geom *g, int nsym_total) {
  return OR_HDR + pad16(4 * OR_NCTX + 2 * (uint64_t)nsym_total) + pad16(4 * (uint64_t)g->R) +
         pad16(4 * (uint64_t)(g->T + 1));
}

/* estimated stream bits: the symbols' information plus every state's cost
 * plus the padding and the metadata */
static double stream_bits(const or_geom *g, double info, int nsym_total) {
  return info + OR_STATE_BITS * (double)(g->S * g->T) + OR_TILE_PAD_BITS * (double)g->T + OR_WORDS_PAD_BITS +
         8.0 * (double)meta_bytes(g, nsym_total);
}

/* the least a stream of this geometry can cost, in bits per element: every
 * state coding nothing */
static double floor_bpp(const or_geom *g) {
  return (OR_STATE_MIN_BITS * (double)(g->S * g->T) + 8.0 * (double)meta_bytes(g, OR_NCTX)) /
         ((double)g->R * (double)g->C);
}

/* ------------------------------------------------------------------------ */
/* Full quantization of the matrix (v laid out row-major, R x Cp).           */
/* ------------------------------------------------------------------------ */
static int quantize_all(const double *x, const or_geom *g, const float *gs, int32_t *v) {
  for (int64_t r = 0; r < g->R; r++)
    for (int64_t k = 0; k < g->vpr; k++) {
      int32_t *vv = v + r * g->Cp + 8 * k;
      quantize_vector(x + r * g->C, g->C, k, gs[r], vv);
      for (int j = 0; j < 8; j++)
        if (!value_in_range(vv[j], g->prob_bits)) return OR_WARN_RAW;
    }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Interleaved rANS over one tile.                                           */
/* Decode order: step s, coordinate j, state q (ascending), for local vector */
/* i = s*S + q when i < n (steps = tile_vecs / S vectors per state).         */
/* Decode: slot = x mod M; x = f*(x >> prob_bits) + slot - c;                */
/*         if x < L: x = (x << 16) | w, w = state q's next word.             */
/* Encode (every state starts at x = L, walking the decode order backwards): */
/*         if x >= f * 2^(27 - prob_bits): emit x & 0xffff, x >>= 16;       */
/*         x = (x / f) * M + (x mod f) + c.                                  */
/* The final encoder state is the decoder's start state, in [2^11, 2^27).    */
/*                                                                           */
/* Tile word layout (16-bit words, little-endian):                          */
/*   S/4 words of pair counts: byte k = words in the region of states 2k,   */
/*     2k+1;                                                                 */
/*   S/4 words of length codes: nibble q (word q/4, bits 4(q%4)..) = W - 12, */
/*     W the bit length of state q's start state;                           */
/*   the start states' low W - 1 bits (the leading one is implied), states  */
/*     ascending, least significant bit first, zero-padded to a whole word; */
/*   region k: state 2k's words in the order it consumes them, then state   */
/*     2k+1's words in reverse order (it reads its region from the end).    */
/* ------------------------------------------------------------------------ */
typedef struct {
  uint16_t *w;
  uint64_t n, cap;
} or_words;

static int words_push(or_words *ws, uint16_t w) {
  if (ws->n == ws->cap) {
    uint64_t nc = ws->cap ? 2 * ws->cap : 1024;
    uint16_t *nw = (uint16_t *)realloc(ws->w, nc * sizeof(uint16_t));
    if (!nw) return OR_ERR_NOMEM;
    ws->w = nw;
    ws->cap = nc;
  }
  ws->w[ws->n++] = w;
  return OR_OK;
}

static int bit_length(uint32_t x) {
  int n = 0;
  while (x) { n++; x >>= 1; }
  return n;
}

/* A bit string of at most 64 states x 26 bits, least significant bit first. */
typedef struct {
  uint16_t w[OR_STATES_DEFAULT * 2];
  int nbits;
} or_bitbuf;

static void bits_put(or_bitbuf *bb, uint32_t value, int nbits) {
  for (int i = 0; i < nbits; i++) {
    if ((value >> i) & 1u) bb->w[bb->nbits >> 4] |= (uint16_t)(1u << (bb->nbits & 15));
    bb->nbits++;
  }
}

/* v: the matrix's lattice coordinates; appends the tile's words to out.
 * Returns OR_WARN_RAW if a pair's word count does not fit its byte. */
static int encode_tile(const or_geom *g, const or_tables *t, const int32_t *v, int64_t tile, or_words *out) {
  int64_t steps = g->tile_vecs / g->S;
  uint32_t M = 1u << g->prob_bits;
  int S = (int)g->S;
  int rc = OR_OK;
  uint32_t x[OR_STATES_DEFAULT];
  or_words rev = {0, 0, 0};
  int32_t *owner = NULL; /* state that emitted each reversed word */
  uint64_t owner_cap = 0;
  int64_t cnt[OR_STATES_DEFAULT], start[OR_STATES_DEFAULT + 1], cur[OR_STATES_DEFAULT];
  uint16_t *lane_words = NULL;
  or_bitbuf bb;
  memset(&bb, 0, sizeof(bb));
  for (int q = 0; q < S; q++) { x[q] = OR_STATE_L; cnt[q] = 0; cur[q] = 0; }
  for (int64_t s = steps - 1; s >= 0; s--)
    for (int j = 7; j >= 0; j--)
      for (int q = S - 1; q >= 0; q--) {
        int64_t vid = tile_vector(g, tile, s * S + q);
        if (vid < 0) continue;
        int64_t r = vid / g->vpr, k = vid % g->vpr;
        int ctx[8];
        int32_t sym[8];
        vector_symbols(v + r * g->Cp + 8 * k, ctx, sym);
        int si = sym[j] - t->smin[ctx[j]];
        uint32_t f = t->freq[ctx[j]][si], c = t->cum[ctx[j]][si];
        uint32_t xs = x[q];
        if ((uint64_t)xs >= ((uint64_t)f << (OR_STATE_TOP - g->prob_bits))) {
          if ((rc = words_push(&rev, (uint16_t)(xs & 0xffffu)))) goto done;
          if (rev.n > owner_cap) {
            owner_cap = rev.cap;
            int32_t *no = (int32_t *)realloc(owner, owner_cap * sizeof(int32_t));
            if (!no) { rc = OR_ERR_NOMEM; goto done; }
            owner = no;
          }
          owner[rev.n - 1] = q;
          xs >>= 16;
        }
        x[q] = (xs / f) * M + (xs % f) + c;
      }
  /* consumption order is the reverse of emission order; split it into
   * per-state lists */
  for (uint64_t k = 0; k < rev.n; k++) cnt[owner[k]]++;
  start[0] = 0;
  for (int q = 0; q < S; q++) start[q + 1] = start[q] + cnt[q];
  lane_words = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(rev.n + 1));
  if (!lane_words) { rc = OR_ERR_NOMEM; goto done; }
  for (uint64_t k = rev.n; k > 0; k--) {
    int32_t q = owner[k - 1];
    lane_words[start[q] + cur[q]++] = rev.w[k - 1];
  }
  /* pair counts */
  for (int q = 0; q < S; q += 4) {
    int64_t lo = cnt[q] + cnt[q + 1], hi = cnt[q + 2] + cnt[q + 3];
    if (lo > 255 || hi > 255) { rc = OR_WARN_RAW; goto done; } /* a count byte cannot hold it: encoding failure */
    if ((rc = words_push(out, (uint16_t)(lo | (hi << 8))))) goto done;
  }
  /* length codes */
  for (int q = 0; q < S; q += 4) {
    uint32_t w = 0;
    for (int i = 0; i < 4; i++) w |= (uint32_t)(bit_length(x[q + i]) - 12) << (4 * i);
    if ((rc = words_push(out, (uint16_t)w))) goto done;
  }
  /* start states below their leading one */
  for (int q = 0; q < S; q++) {
    int W = bit_length(x[q]);
    bits_put(&bb, x[q], W - 1);
  }
  for (int k = 0; k < (bb.nbits + 15) / 16; k++)
    if ((rc = words_push(out, bb.w[k]))) goto done;
  /* pair regions */
  for (int q = 0; q < S; q += 2) {
    for (int64_t k = 0; k < cnt[q]; k++)
      if ((rc = words_push(out, lane_words[start[q] + k]))) goto done;
    for (int64_t k = cnt[q + 1] - 1; k >= 0; k--)
      if ((rc = words_push(out, lane_words[start[q + 1] + k]))) goto done;
  }
done:
  free(rev.w);
  free(owner);
  free(lane_words);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Stream writer.                                                            */
/* header(128) | tables | scales f32[R] | tile word offsets u32[T+1] |       */
/* words u16[n_words]; sections 16-aligned.  The header's states-section    */
/* offset (byte 80) is 0: start states live in the tiles.                   */
/* ------------------------------------------------------------------------ */
static int write_lattice_blob(const or_geom *g, int dtype, double a, double target, const or_tables *t,
                              const float *gs, const uint32_t *toff, const or_words *ws, uint8_t **blob,
                              size_t *nbytes) {
  int nsym = tables_total_nsym(t);
  uint64_t o_tab = OR_HDR;
  uint64_t o_sc = o_tab + pad16(4 * OR_NCTX + 2 * (uint64_t)nsym);
  uint64_t o_to = o_sc + pad16(4 * (uint64_t)g->R);
  uint64_t o_w = o_to + pad16(4 * (uint64_t)(g->T + 1));
  uint64_t total = o_w + pad16(2 * ws->n);
  uint8_t *b = (uint8_t *)calloc(total, 1);
  if (!b) return OR_ERR_NOMEM;
  put_u32(b + 0, OR_MAGIC);
  put_u16(b + 4, OR_VERSION);
  put_u16(b + 6, OR_HDR);
  b[8] = 0; /* lattice-rANS */
  b[9] = (uint8_t)dtype;
  b[10] = (uint8_t)g->prob_bits;
  b[11] = OR_NCTX;
  put_u32(b + 12, (uint32_t)g->tile_vecs);
  put_u32(b + 16, (uint32_t)g->S);
  put_u32(b + 20, (uint32_t)g->T);
  put_u64(b + 24, (uint64_t)g->R);
  put_u64(b + 32, (uint64_t)g->C);
  put_u64(b + 40, (uint64_t)g->Cp);
  put_f64(b + 48, a);
  put_f64(b + 56, target);
  put_u64(b + 64, o_tab);
  put_u64(b + 72, o_sc);
  put_u64(b + 80, 0);
  put_u64(b + 88, o_to);
  put_u64(b + 96, o_w);
  put_u64(b + 104, ws->n);
  put_u64(b + 112, total);
  b[120] = (uint8_t)g->layout;
  uint8_t *p = b + o_tab;
  for (int c = 0; c < OR_NCTX; c++) {
    put_u16(p + 4 * c, (uint32_t)(uint16_t)(int16_t)t->smin[c]);
    put_u16(p + 4 * c + 2, (uint32_t)t->nsym[c]);
  }
  p += 4 * OR_NCTX;
  for (int c = 0; c < OR_NCTX; c++)
    for (int s = 0; s < t->nsym[c]; s++) {
      put_u16(p, t->freq[c][s]);
      p += 2;
    }
  for (int64_t r = 0; r < g->R; r++) put_f32(b + o_sc + 4 * r, gs[r]);
  for (int64_t i = 0; i <= g->T; i++) put_u32(b + o_to + 4 * i, toff[i]);
  for (uint64_t i = 0; i < ws->n; i++) put_u16(b + o_w + 2 * i, ws->w[i]);
  *blob = b;
  *nbytes = (size_t)total;
  return OR_OK;
}

static int write_raw_blob(int64_t R, int64_t C, int dtype, double target, const void *src,
                          uint8_t **blob, size_t *nbytes) {
  uint64_t payload = (uint64_t)R * (uint64_t)C * (uint64_t)esize_of(dtype);
  uint64_t total = OR_HDR + pad16(payload);
  uint8_t *b = (uint8_t *)calloc(total, 1);
  if (!b) return OR_ERR_NOMEM;
  put_u32(b + 0, OR_MAGIC);
  put_u16(b + 4, OR_VERSION);
  put_u16(b + 6, OR_HDR);
  b[8] = 1; /* raw */
  b[9] = (uint8_t)dtype;
  put_u64(b + 24, (uint64_t)R);
  put_u64(b + 32, (uint64_t)C);
  put_u64(b + 40, (uint64_t)C);
  put_f64(b + 56, target);
  put_u64(b + 96, OR_HDR);
  put_u64(b + 112, total);
  memcpy(b + OR_HDR, src, payload);
  *blob = b;
  *nbytes = (size_t)total;
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Full compression at a fixed lattice scale a.                              */
/* ------------------------------------------------------------------------ */
static long or_encodes; /* full encodes (compress_at calls) since the last or_compress began */

static int compress_at(const double *x, const or_geom *g, int dtype, double a, double target,
                       uint8_t **blob, size_t *nbytes) {
  int rc;
  or_encodes++;
  float *gs = (float *)malloc(sizeof(float) * (size_t)g->R);
  int32_t *v = (int32_t *)malloc(sizeof(int32_t) * (size_t)(g->R * g->Cp));
  uint32_t *toff = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(g->T + 1));
  or_hist *h = (or_hist *)calloc(1, sizeof(or_hist));
  or_tables t;
  memset(&t, 0, sizeof(t));
  or_words ws = {0, 0, 0};
  if (!gs || !v || !toff || !h) { rc = OR_ERR_NOMEM; goto done; }
  for (int64_t r = 0; r < g->R; r++) gs[r] = stored_scale(row_rms(x + r * g->C, g->C), a);
  rc = quantize_all(x, g, gs, v);
  if (rc) goto done;
  for (int64_t vid = 0; vid < g->n_vec; vid++) {
    int ctx[8];
    int32_t sym[8];
    vector_symbols(v + (vid / g->vpr) * g->Cp + 8 * (vid % g->vpr), ctx, sym);
    for (int j = 0; j < 8; j++) h->cnt[ctx[j]][sym[j] + OR_SYM_OFF]++;
  }
  rc = tables_from_hist(h, g->prob_bits, &t);
  /* a context that needs more than 2^prob_bits symbols cannot be coded: an
   * encoding failure, like values outside the stream's range (the sampled
   * estimate may have seen fewer symbols than the whole matrix holds) */
  if (rc == OR_ERR_TARGET) rc = OR_WARN_RAW;
  if (rc) goto done;
  for (int64_t tile = 0; tile < g->T; tile++) {
    if (ws.n > 0xffffffffu) { rc = OR_ERR_SHAPE; goto done; }
    toff[tile] = (uint32_t)ws.n;
    rc = encode_tile(g, &t, v, tile, &ws);
    if (rc) goto done;
  }
  if (ws.n > 0xffffffffu) { rc = OR_ERR_SHAPE; goto done; }
  toff[g->T] = (uint32_t)ws.n;
  rc = write_lattice_blob(g, dtype, a, target, &t, gs, toff, &ws, blob, nbytes);
done:
  free(gs);
  free(v);
  free(toff);
  free(h);
  free(ws.w);
  tables_free(&t);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Sampled storage estimate (the pages' resolution selection without         */
/* repeated full-stream encoding).  n = min(n_vec, sample_vecs) vectors at   */
/* indices floor(k * n_vec / n) + phase, phase = seed mod floor(n_vec / n);  */
/* tables are built from the sample alone;                                   */
/* bits = (n_vec / n) * sum_s c_s (prob_bits - log2 f_s)                     */
/*        + 18.5 per state + padding + 8 * (header, tables, scales, offsets) */
/* (stream_bits above).  Out-of-range lattice values give +inf.             */
/* ------------------------------------------------------------------------ */
typedef struct {
  int64_t vecs;  /* sample size (vectors) */
  uint64_t seed; /* sample phase */
} or_sample;

static int64_t sample_size(const or_geom *g, const or_sample *sp) {
  return g->n_vec < sp->vecs ? g->n_vec : sp->vecs;
}

/* vector index of sample k of n */
static int64_t sample_vid(const or_geom *g, const or_sample *sp, int64_t k, int64_t n) {
  uint64_t stride = (uint64_t)g->n_vec / (uint64_t)n;
  uint64_t phase = sp->seed % stride;
  return (int64_t)(((uint64_t)k * (uint64_t)g->n_vec) / (uint64_t)n + phase);
}

static double info_bits(const or_hist *h, const or_tables *t, int prob_bits) {
  double info = 0.0;
  for (int c = 0; c < OR_NCTX; c++)
    for (int s = 0; s < t->nsym[c]; s++) {
      uint64_t cnt = (t->smin[c] + s + OR_SYM_OFF < OR_SYM_SPAN) ? h->cnt[c][t->smin[c] + s + OR_SYM_OFF] : 0;
      if (cnt) info += (double)cnt * ((double)prob_bits - log2((double)t->freq[c][s]));
    }
  return info;
}

double or_estimate_bpp_rows(const double *x, const double *rms, const or_geom *g, const or_sample *sp, double a) {
  int64_t n = sample_size(g, sp);
  or_hist *h = (or_hist *)calloc(1, sizeof(or_hist));
  if (!h) return NAN;
  for (int64_t k = 0; k < n; k++) {
    int64_t vid = sample_vid(g, sp, k, n);
    int64_t r = vid / g->vpr, kk = vid % g->vpr;
    int32_t v[8];
    int ctx[8];
    int32_t sym[8];
    quantize_vector(x + r * g->C, g->C, kk, stored_scale(rms[r], a), v);
    for (int j = 0; j < 8; j++)
      if (!value_in_range(v[j], g->prob_bits)) { free(h); return INFINITY; }
    vector_symbols(v, ctx, sym);
    for (int j = 0; j < 8; j++) h->cnt[ctx[j]][sym[j] + OR_SYM_OFF]++;
  }
  or_tables t;
  int rc = tables_from_hist(h, g->prob_bits, &t);
  if (rc) { tables_free(&t); free(h); return INFINITY; }
  double info = info_bits(h, &t, g->prob_bits) * ((double)g->n_vec / (double)n);
  double bits = stream_bits(g, info, tables_total_nsym(&t));
  tables_free(&t);
  free(h);
  return bits / ((double)g->R * (double)g->C);
}

/* Estimate with the exact tables of the whole matrix at scale a: every vector
 * quantized and histogrammed, no entropy coding.  Same formula as the sampled
 * estimate with a sample of every vector. */
static double estimate_bpp_full(const double *x, const or_geom *g, double a) {
  float *gs = (float *)malloc(sizeof(float) * (size_t)g->R);
  int32_t *v = (int32_t *)malloc(sizeof(int32_t) * (size_t)(g->R * g->Cp));
  or_hist *h = (or_hist *)calloc(1, sizeof(or_hist));
  double result = NAN;
  or_tables t;
  memset(&t, 0, sizeof(t));
  if (!gs || !v || !h) goto done;
  for (int64_t r = 0; r < g->R; r++) gs[r] = stored_scale(row_rms(x + r * g->C, g->C), a);
  if (quantize_all(x, g, gs, v) != OR_OK) { result = INFINITY; goto done; }
  for (int64_t vid = 0; vid < g->n_vec; vid++) {
    int ctx[8];
    int32_t sym[8];
    vector_symbols(v + (vid / g->vpr) * g->Cp + 8 * (vid % g->vpr), ctx, sym);
    for (int j = 0; j < 8; j++) h->cnt[ctx[j]][sym[j] + OR_SYM_OFF]++;
  }
  if (tables_from_hist(h, g->prob_bits, &t) != OR_OK) { result = INFINITY; goto done; }
  result = stream_bits(g, info_bits(h, &t, g->prob_bits), tables_total_nsym(&t)) / ((double)g->R * (double)g->C);
done:
  tables_free(&t);
  free(gs);
  free(v);
  free(h);
  return result;
}

/* bisection on log2(a) toward the target; returns the a whose estimate is
 * closest to the target among those evaluated */
typedef double (*or_rate_fn)(void *ctx, double a);

static double select_scale(or_rate_fn fn, void *ctx, double target, double *best_est) {
  const double two_pi_e = 17.079468445347132; /* 2*pi*e */
  double la0 = 0.5 * log2(two_pi_e) - target;
  double lo = la0 - 1.0, hi = la0 + 1.0;
  double best_la = la0, best_err = INFINITY, best_e = INFINITY;
#define OR_TRY(la, e)                                                        \
  do {                                                                       \
    double err_ = fabs((e) - target);                                        \
    if (err_ < best_err) { best_err = err_; best_la = (la); best_e = (e); }  \
  } while (0)
  double e_lo = fn(ctx, exp2(lo));
  OR_TRY(lo, e_lo);
  for (int k = 0; k < 30 && e_lo < target; k++) {
    lo -= 2.0;
    e_lo = fn(ctx, exp2(lo));
    OR_TRY(lo, e_lo);
  }
  double e_hi = fn(ctx, exp2(hi));
  OR_TRY(hi, e_hi);
  for (int k = 0; k < 30 && e_hi > target; k++) {
    hi += 2.0;
    e_hi = fn(ctx, exp2(hi));
    OR_TRY(hi, e_hi);
  }
  for (int it = 0; it < 40; it++) {
    double mid = 0.5 * (lo + hi);
    double e = fn(ctx, exp2(mid));
    OR_TRY(mid, e);
    if (fabs(e - target) <= 5e-4 * target) break;
    if (e > target) lo = mid;
    else hi = mid;
  }
#undef OR_TRY
  *best_est = best_e;
  return exp2(best_la);
}

typedef struct {
  const double *x;
  const double *rms;
  const or_geom *g;
  const or_sample *sp;
  int dtype;
  double target;
} or_sel_ctx;

static double rate_sampled(void *vctx, double a) {
  or_sel_ctx *c = (or_sel_ctx *)vctx;
  return or_estimate_bpp_rows(c->x, c->rms, c->g, c->sp, a);
}

/* exact rate: a full compression per probe (slow; used to pin the estimate) */
static double rate_exact(void *vctx, double a) {
  or_sel_ctx *c = (or_sel_ctx *)vctx;
  uint8_t *b = NULL;
  size_t nb = 0;
  int rc = compress_at(c->x, c->g, c->dtype, a, c->target, &b, &nb);
  free(b);
  if (rc == OR_WARN_RAW) return INFINITY;
  if (rc) return NAN;
  return 8.0 * (double)nb / ((double)c->g->R * (double)c->g->C);
}

/* ------------------------------------------------------------------------ */
/* Public entry points (ctypes)                                              */
/* ------------------------------------------------------------------------ */
static int check_input(const double *x, int64_t R, int64_t C, int dtype, double target) {
  if (!x) return OR_ERR_ARG;
  if (dtype < 0 || dtype > 3) return OR_ERR_ARG;
  if (R <= 0 || C <= 0) return OR_ERR_SHAPE;
  for (int64_t i = 0; i < R * C; i++)
    if (!isfinite(x[i])) return OR_ERR_NONFINITE;
  if (!isfinite(target) || target < 0.001) return OR_ERR_TARGET;
  if (esize_of(dtype) == 2 && target > 11.0) return OR_ERR_TARGET;
  if (esize_of(dtype) == 1 && target >= 8.0) return OR_ERR_TARGET;
  return OR_OK;
}

/*
 * Compress an R x C matrix given as f64 values (widened exactly from the
 * container dtype) plus the container's own bytes (for a raw fallback).
 *   fixed_a > 0      : this lattice resolution, no rate selection;
 *   n_states         : 0 (choose), 16 or 64 rANS states per tile;
 *   tile_vecs        : 0 (choose), 512 or 1024 E8 vectors per tile;
 *   sample_vecs      : 0 (65536) or the rate estimate's sample size;
 *   seed             : the sample's phase (vectors past each stride point);
 *   exact_select != 0: select with a full encode per probe instead of the
 *                      sampled estimate (slow; pins the estimate);
 *   layout           : OR_LAYOUT_ROWS or OR_LAYOUT_BLOCKS (64 x 64 weight
 *                      blocks; BF16, C % 8 == 0, 64 states, 512 vectors).
 * With the state count chosen, tiles have 64 states, or 16 when a
 * target-selected stream's target is less than 4x the least a 64-state stream
 * costs (64 states would spend over a quarter of the bits on their overhead).  With the tile size chosen, 64-state tiles hold 512 vectors in
 * matrices of fewer than 2^22 vectors (twice the tiles, so twice the states
 * decoding in parallel) and 1024 in larger ones; 16-state tiles hold 512, or
 * 1024 when the target lies below 1.1x the least 512 allow.
 * Exactly one full encode runs for a lattice stream (or_last_encode_count).
 */
int or_compress(const double *x, const void *src_bytes, int64_t R, int64_t C, int dtype, double target,
                double fixed_a, int n_states, int64_t tile_vecs, int64_t sample_vecs, uint64_t seed, int prob_bits,
                int exact_select, int layout, uint8_t **blob, size_t *nbytes, double *a_out) {
  or_encodes = 0;
  int rc = check_input(x, R, C, dtype, target);
  if (rc) return rc;
  if (layout != OR_LAYOUT_ROWS && layout != OR_LAYOUT_BLOCKS) return OR_ERR_ARG;
  if (layout == OR_LAYOUT_BLOCKS) {
    /* the blocks layout feeds a BF16 matrix multiply: BF16 containers, whole
     * vectors per row, 64 states and 512 vectors per tile */
    if (dtype != OR_BF16 || (n_states != 0 && n_states != 64) || (tile_vecs != 0 && tile_vecs != 512))
      return OR_ERR_ARG;
    if (C % 8 != 0) return OR_ERR_SHAPE;
    n_states = 64;
    tile_vecs = 512;
  }
  if ((n_states != 0 && n_states != 16 && n_states != 64) ||
      (tile_vecs != 0 && tile_vecs != 512 && tile_vecs != 1024) || sample_vecs < 0 || prob_bits < 8 ||
      prob_bits > 11 || !blob || !nbytes)
    return OR_ERR_ARG;
  if (R * ((C + 7) / 8) >= ((int64_t)1 << 31)) return OR_ERR_SHAPE;
  const int chosen = !(fixed_a > 0.0);
  or_geom g;
  if (n_states == 0) {
    int64_t tv = tile_vecs ? tile_vecs : (R * ((C + 7) / 8) < OR_SMALL_MATRIX_VECS ? 512 : 1024);
    geom_init(&g, R, C, OR_STATES_DEFAULT, tv, prob_bits, layout);
    n_states = (chosen && target < 4.0 * floor_bpp(&g)) ? OR_STATES_LOW : OR_STATES_DEFAULT;
  }
  if (tile_vecs == 0) {
    if (n_states == OR_STATES_DEFAULT) {
      tile_vecs = R * ((C + 7) / 8) < OR_SMALL_MATRIX_VECS ? 512 : 1024;
    } else {
      geom_init(&g, R, C, n_states, 512, prob_bits, layout);
      tile_vecs = (chosen && target < 1.1 * floor_bpp(&g)) ? 1024 : 512;
    }
  }
  geom_init(&g, R, C, n_states, tile_vecs, prob_bits, layout);
  or_sample sp = {sample_vecs ? sample_vecs : OR_SAMPLE_VECS, seed};
  double a = fixed_a;
  double *rms = NULL;
  or_sel_ctx sc = {x, NULL, &g, &sp, dtype, target};
  if (chosen) {
    rms = (double *)malloc(sizeof(double) * (size_t)R);
    if (!rms) return OR_ERR_NOMEM;
    for (int64_t r = 0; r < R; r++) rms[r] = row_rms(x + r * C, C);
    sc.rms = rms;
    /* targets below the fixed per-state overhead cannot be met */
    if (target < 1.02 * floor_bpp(&g)) { free(rms); return OR_ERR_TARGET; }
    double best_est = INFINITY;
    a = select_scale(exact_select ? rate_exact : rate_sampled, &sc, target, &best_est);
    if (exact_select) or_encodes = 0; /* the probes' encodes are the exact selection's, not the stream's */
    /* no resolution reaches the target within 2% (the lattice values would
     * leave the stream's value range first): an encoding failure */
    if (!(fabs(best_est - target) <= 0.02 * target)) {
      free(rms);
      if (a_out) *a_out = a;
      if (!src_bytes) return OR_ERR_ARG;
      rc = write_raw_blob(R, C, dtype, target, src_bytes, blob, nbytes);
      return rc ? rc : OR_WARN_RAW;
    }
    /* the sample misses rare symbols that the full tables must still give a
     * frequency of at least 1; one histogram of the whole matrix at the chosen
     * scale (no entropy coding) measures that bias, and when it exceeds 0.5%
     * the sampled bisection runs again toward the target minus the bias.  The
     * bias changes with the scale, so this repeats (at most three bisections)
     * until the whole-matrix estimate is within 0.5% of the target. */
    if (!exact_select) {
      double full = estimate_bpp_full(x, &g, a);
      if (isfinite(full) && !(fabs(full - target) <= 0.005 * target)) {
        double est = best_est;
        for (int it = 0; it < 3; it++) {
          a = select_scale(rate_sampled, &sc, target - (full - est), &est);
          if (it == 2) break;
          full = estimate_bpp_full(x, &g, a);
          if (!isfinite(full) || fabs(full - target) <= 0.005 * target) break;
        }
      }
    }
  }
  if (a_out) *a_out = a;
  rc = compress_at(x, &g, dtype, a, target, blob, nbytes);
  free(rms);
  uint64_t raw_total = OR_HDR + pad16((uint64_t)R * (uint64_t)C * (uint64_t)esize_of(dtype));
  /* with the resolution chosen from the target, a lattice stream no smaller
   * than the raw container is an encoding failure; a fixed resolution keeps
   * the lattice stream */
  if (rc == OR_OK && chosen && (uint64_t)*nbytes >= raw_total) {
    free(*blob);
    *blob = NULL;
    rc = OR_WARN_RAW;
  }
  if (rc == OR_WARN_RAW) {
    if (!src_bytes) return OR_ERR_ARG;
    rc = write_raw_blob(R, C, dtype, target, src_bytes, blob, nbytes);
    return rc ? rc : OR_WARN_RAW;
  }
  return rc;
}

/* full encodes the last or_compress ran (1 for a lattice stream, also after
 * an exact selection, whose probes are not counted) */
long or_last_encode_count(void) { return or_encodes; }

double or_estimate_bpp(const double *x, int64_t R, int64_t C, double a, int n_states, int64_t tile_vecs,
                       int64_t sample_vecs, uint64_t seed, int prob_bits, int layout) {
  or_geom g;
  geom_init(&g, R, C, n_states, tile_vecs, prob_bits, layout);
  or_sample sp = {sample_vecs ? sample_vecs : OR_SAMPLE_VECS, seed};
  double *rms = (double *)malloc(sizeof(double) * (size_t)R);
  if (!rms) return NAN;
  for (int64_t r = 0; r < R; r++) rms[r] = row_rms(x + r * C, C);
  double e = or_estimate_bpp_rows(x, rms, &g, &sp, a);
  free(rms);
  return e;
}

void or_free(void *p) { free(p); }

/* direct quantize-and-reconstruct coordinates (no entropy coding): v for
 * every padded coordinate and the stored scales g, at lattice scale a */
int or_quantize_matrix(const double *x, int64_t R, int64_t C, double a, int prob_bits, float *g_out,
                       int32_t *v_out) {
  if (!x || R <= 0 || C <= 0 || !g_out || !v_out) return OR_ERR_ARG;
  or_geom g;
  geom_init(&g, R, C, 64, 1024, prob_bits, OR_LAYOUT_ROWS);
  for (int64_t r = 0; r < R; r++) g_out[r] = stored_scale(row_rms(x + r * C, C), a);
  for (int64_t r = 0; r < R; r++)
    for (int64_t k = 0; k < g.vpr; k++) quantize_vector(x + r * C, C, k, g_out[r], v_out + r * g.Cp + 8 * k);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Stream reader and decoder                                                 */
/* ------------------------------------------------------------------------ */
typedef struct {
  int method, dtype;
  or_geom g;
  double a, target;
  uint64_t o_tab, o_sc, o_to, o_w, n_words, total;
} or_header;

/* [off, off + size) inside [0, nb), written so that no sum can wrap */
static int span_ok(uint64_t off, uint64_t size, uint64_t nb) { return off <= nb && size <= nb - off; }

/* Header and section table.  Rows and columns are capped below 2^31 (and
 * their product below 2^40) before any product is formed, and every section
 * bound is checked as an offset and a size against the stream length, so a
 * corrupt header cannot make a check overflow. */
static int parse_header(const uint8_t *b, size_t nb, or_header *h) {
  if (!b || nb < OR_HDR) return OR_ERR_FORMAT;
  if (get_u32(b) != OR_MAGIC || get_u16(b + 4) != OR_VERSION || get_u16(b + 6) != OR_HDR) return OR_ERR_FORMAT;
  h->method = b[8];
  h->dtype = b[9];
  if (h->dtype > 3 || h->method > 1) return OR_ERR_FORMAT;
  uint64_t R = get_u64(b + 24), C = get_u64(b + 32);
  if (R == 0 || C == 0 || R >= ((uint64_t)1 << 31) || C >= ((uint64_t)1 << 31) || R * C >= ((uint64_t)1 << 40))
    return OR_ERR_FORMAT;
  h->total = get_u64(b + 112);
  if (h->total != nb) return OR_ERR_FORMAT;
  h->target = get_f64(b + 56);
  if (h->method == 1) {
    geom_init(&h->g, (int64_t)R, (int64_t)C, 64, 1024, 10, OR_LAYOUT_ROWS);
    h->o_w = get_u64(b + 96);
    if (h->o_w != OR_HDR || !span_ok(OR_HDR, R * C * (uint64_t)esize_of(h->dtype), nb)) return OR_ERR_FORMAT;
    return OR_OK;
  }
  int pb = b[10];
  if (pb < 8 || pb > 11 || b[11] != OR_NCTX) return OR_ERR_FORMAT;
  int64_t S = get_u32(b + 16), TV = get_u32(b + 12);
  if ((S != 16 && S != 64) || (TV != 512 && TV != 1024)) return OR_ERR_FORMAT;
  if (R * ((C + 7) / 8) >= ((uint64_t)1 << 31)) return OR_ERR_FORMAT;
  int layout = b[120];
  if (layout > OR_LAYOUT_BLOCKS) return OR_ERR_FORMAT;
  if (layout == OR_LAYOUT_BLOCKS && (S != 64 || TV != 512 || C % 8 != 0 || h->dtype != OR_BF16)) return OR_ERR_FORMAT;
  geom_init(&h->g, (int64_t)R, (int64_t)C, S, TV, pb, layout);
  if ((int64_t)get_u64(b + 40) != h->g.Cp || (int64_t)get_u32(b + 20) != h->g.T) return OR_ERR_FORMAT;
  h->a = get_f64(b + 48);
  h->o_tab = get_u64(b + 64);
  h->o_sc = get_u64(b + 72);
  h->o_to = get_u64(b + 88);
  h->o_w = get_u64(b + 96);
  h->n_words = get_u64(b + 104);
  uint64_t T = (uint64_t)h->g.T; /* below 2^22 here */
  if (h->o_tab != OR_HDR || !span_ok(h->o_tab, 4 * OR_NCTX, nb) || get_u64(b + 80) != 0) return OR_ERR_FORMAT;
  if (!span_ok(h->o_sc, 4 * R, nb) || h->o_sc < h->o_tab + 4 * OR_NCTX ||
      !span_ok(h->o_to, 4 * (T + 1), nb) || h->o_to < h->o_sc + 4 * R ||
      h->n_words > nb || !span_ok(h->o_w, 2 * h->n_words, nb) || h->o_w < h->o_to + 4 * (T + 1))
    return OR_ERR_FORMAT;
  return OR_OK;
}

static int read_tables(const uint8_t *b, const or_header *h, or_tables *t) {
  memset(t, 0, sizeof(*t));
  const uint8_t *p = b + h->o_tab + 4 * OR_NCTX;
  uint32_t M = 1u << h->g.prob_bits;
  for (int c = 0; c < OR_NCTX; c++) {
    t->smin[c] = (int16_t)get_u16(b + h->o_tab + 4 * c);
    t->nsym[c] = (int)get_u16(b + h->o_tab + 4 * c + 2);
    if (p + 2 * (size_t)t->nsym[c] > b + h->o_sc) return OR_ERR_FORMAT;
    t->freq[c] = (uint32_t *)calloc((size_t)t->nsym[c] + 1, sizeof(uint32_t));
    t->cum[c] = (uint32_t *)calloc((size_t)t->nsym[c] + 2, sizeof(uint32_t));
    if (!t->freq[c] || !t->cum[c]) return OR_ERR_NOMEM;
    for (int s = 0; s < t->nsym[c]; s++) {
      t->freq[c][s] = get_u16(p);
      p += 2;
      t->cum[c][s + 1] = t->cum[c][s] + t->freq[c][s];
    }
    if (t->nsym[c] > 0 && t->cum[c][t->nsym[c]] != M) return OR_ERR_FORMAT;
  }
  return OR_OK;
}

/* Decode tiles [t0, t1) into v (R x Cp lattice coordinates, int32). */
static int decode_lattice_tiles(const uint8_t *b, const or_header *h, int32_t *v, int64_t t0, int64_t t1) {
  or_tables t;
  int rc = read_tables(b, h, &t);
  if (rc) { tables_free(&t); return rc; }
  const or_geom *g = &h->g;
  const int S = (int)g->S;
  uint32_t M = 1u << g->prob_bits;
  int64_t steps = g->tile_vecs / S;
  uint32_t x[OR_STATES_DEFAULT];
  int64_t fwd[OR_STATES_DEFAULT / 2], bwd[OR_STATES_DEFAULT / 2]; /* next word of states 2k and 2k+1 */
  int32_t vb[OR_STATES_DEFAULT], zp[OR_STATES_DEFAULT];           /* coset bit, running z sum */
  const uint8_t *words = b + h->o_w;
  for (int64_t tile = t0; tile < t1; tile++) {
    int64_t wp = get_u32(b + h->o_to + 4 * tile);
    int64_t wend = get_u32(b + h->o_to + 4 * (tile + 1));
    int64_t hw = S / 2; /* words of pair counts and length codes */
    if (wend < wp || wend > (int64_t)h->n_words || wend - wp < hw) { rc = OR_ERR_FORMAT; goto done; }
    /* start states: length codes, then the bits below each leading one */
    int64_t bitpos = 0, bit0 = 2 * (wp + hw);
    for (int q = 0; q < S; q++) {
      int W = (int)((get_u16(words + 2 * (wp + S / 4 + q / 4)) >> (4 * (q % 4))) & 15u) + 12;
      uint32_t val = 1u << (W - 1);
      for (int i = 0; i < W - 1; i++, bitpos++) {
        int64_t byte = bit0 + bitpos / 8;
        if (byte >= 2 * wend) { rc = OR_ERR_FORMAT; goto done; }
        if ((words[byte] >> (bitpos % 8)) & 1u) val |= 1u << i;
      }
      x[q] = val;
    }
    /* pair regions after the start bits' whole words */
    int64_t r0 = wp + hw + (bitpos + 15) / 16;
    for (int k = 0; k < S / 2; k++) {
      int64_t cnt = words[2 * wp + k];
      fwd[k] = r0;
      r0 += cnt;
      bwd[k] = r0 - 1;
    }
    if (r0 != wend) { rc = OR_ERR_FORMAT; goto done; }
    for (int64_t s = 0; s < steps; s++)
      for (int j = 0; j < 8; j++) {
        for (int q = 0; q < S; q++) {
          int64_t vid = tile_vector(g, tile, s * S + q);
          if (vid < 0) continue;
          int ctx;
          if (j == 0) ctx = 0;
          else if (j < 7) ctx = 1 + vb[q];
          else ctx = 3 + 2 * vb[q] + (zp[q] & 1);
          if (t.nsym[ctx] == 0) { rc = OR_ERR_FORMAT; goto done; }
          uint32_t slot = x[q] & (M - 1);
          int si = 0;
          while (!(t.cum[ctx][si] <= slot && slot < t.cum[ctx][si + 1])) si++;
          x[q] = t.freq[ctx][si] * (x[q] >> g->prob_bits) + slot - t.cum[ctx][si];
          if (x[q] < OR_STATE_L) {
            int k = q / 2;
            if (fwd[k] > bwd[k]) { rc = OR_ERR_FORMAT; goto done; } /* the pair's region is used up */
            int64_t at = (q % 2 == 0) ? fwd[k]++ : bwd[k]--;
            x[q] = (x[q] << 16) | get_u16(words + 2 * at);
          }
          int32_t sym = t.smin[ctx] + si;
          int32_t *vv = v + (vid / g->vpr) * g->Cp + 8 * (vid % g->vpr);
          if (j == 0) {
            vv[0] = sym;
            vb[q] = sym & 1;
            zp[q] = (sym - vb[q]) / 2;
          } else {
            vv[j] = symbol_value(ctx, sym, vb[q], zp[q] & 1);
            if (j < 7) zp[q] += sym;
          }
        }
      }
    /* every state ends at L (states without vectors start there), and every
     * pair has used its whole region */
    for (int q = 0; q < S; q++)
      if (x[q] != OR_STATE_L) { rc = OR_ERR_FORMAT; goto done; }
    for (int k = 0; k < S / 2; k++)
      if (fwd[k] != bwd[k] + 1) { rc = OR_ERR_FORMAT; goto done; }
  }
done:
  tables_free(&t);
  return rc;
}

/* Decode every tile into v (R x Cp lattice coordinates, int32). */
static int decode_lattice(const uint8_t *b, const or_header *h, int32_t *v) {
  return decode_lattice_tiles(b, h, v, 0, h->g.T);
}

/* lattice coordinates v (int16, R x Cp) of a lattice stream */
int or_decode_symbols(const uint8_t *b, size_t nb, int16_t *v_out) {
  or_header h;
  int rc = parse_header(b, nb, &h);
  if (rc) return rc;
  if (h.method != 0 || !v_out) return OR_ERR_ARG;
  int32_t *v = (int32_t *)malloc(sizeof(int32_t) * (size_t)(h.g.R * h.g.Cp));
  if (!v) return OR_ERR_NOMEM;
  rc = decode_lattice(b, &h, v);
  if (!rc)
    for (int64_t i = 0; i < h.g.R * h.g.Cp; i++) v_out[i] = (int16_t)v[i];
  free(v);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Container conversions from f32, written from the format definitions.      */
/* ------------------------------------------------------------------------ */
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16: top 16 bits of binary32, round to nearest, ties to even */
uint16_t or_f32_to_bf16(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/*
 * Round a non-negative finite value to a binary format with `mbits` stored
 * mantissa bits and minimum normal exponent emin, to nearest with ties to
 * even; subnormals are kept.  Returns the rounded value as an f64.
 */
static double round_to_format(double m, int mbits, int emin) {
  if (m == 0.0) return 0.0;
  int e;
  frexp(m, &e);       /* m = fr * 2^e with fr in [0.5, 1) */
  int exp = e - 1;    /* m = 1.x * 2^exp */
  if (exp < emin) exp = emin;
  double quantum = ldexp(1.0, exp - mbits);
  double q = m / quantum;           /* exact: power-of-two scaling */
  double r = nearbyint(q);          /* ties to even */
  return r * quantum;
}

/* IEEE binary16: 10 mantissa bits, emin = -14, max 65504, overflow -> inf */
uint16_t or_f32_to_f16(float f) {
  uint32_t u = f32_bits(f);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);
  double m = fabs((double)f);
  if (isinf(m)) return (uint16_t)(sign | 0x7c00u);
  double r = round_to_format(m, 10, -14);
  if (r >= 65520.0 || r > 65504.0) return (uint16_t)(sign | 0x7c00u);
  if (r == 0.0) return sign;
  int e;
  double fr = frexp(r, &e);
  int exp = e - 1;
  if (exp < -14) { /* subnormal: r = k * 2^-24 */
    uint16_t k = (uint16_t)(r / ldexp(1.0, -24));
    return (uint16_t)(sign | k);
  }
  uint16_t mant = (uint16_t)((fr * 2.0 - 1.0) * 1024.0);
  return (uint16_t)(sign | ((uint16_t)(exp + 15) << 10) | mant);
}

/* OCP FP8 E4M3FN: 3 mantissa bits, bias 7, emin = -6, max 448, no inf.
 * Values are first clamped to [-448, 448] (saturating conversion). */
uint8_t or_f32_to_e4m3fn(float f) {
  uint32_t u = f32_bits(f);
  uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint8_t)(sign | 0x7f);
  double m = fabs((double)f);
  if (m > 448.0) m = 448.0;
  double r = round_to_format(m, 3, -6);
  if (r > 448.0) r = 448.0;
  if (r == 0.0) return sign;
  int e;
  double fr = frexp(r, &e);
  int exp = e - 1;
  if (exp < -6) { /* subnormal: r = k * 2^-9 */
    uint8_t k = (uint8_t)(r / ldexp(1.0, -9));
    return (uint8_t)(sign | k);
  }
  uint8_t mant = (uint8_t)((fr * 2.0 - 1.0) * 8.0);
  return (uint8_t)(sign | ((uint8_t)(exp + 7) << 3) | mant);
}

/* symmetric INT8 code: round half to even, clamp to [-127, 127] */
int8_t or_f32_to_int8(float f) {
  double r = nearbyint((double)f);
  if (r > 127.0) r = 127.0;
  if (r < -127.0) r = -127.0;
  return (int8_t)r;
}

/* y = f32(f32(v) * g_r), converted to the container */
static void store_value(void *out, int dtype, int64_t idx, int32_t v, float g) {
  float y = (float)v * g;
  switch (dtype) {
    case OR_BF16: ((uint16_t *)out)[idx] = or_f32_to_bf16(y); break;
    case OR_FP16: ((uint16_t *)out)[idx] = or_f32_to_f16(y); break;
    case OR_FP8: ((uint8_t *)out)[idx] = or_f32_to_e4m3fn(y); break;
    default: ((int8_t *)out)[idx] = or_f32_to_int8(y); break;
  }
}

/* Decompress into the container dtype, R x C row-major. */
int or_decompress(const uint8_t *b, size_t nb, void *out) {
  or_header h;
  int rc = parse_header(b, nb, &h);
  if (rc) return rc;
  if (!out) return OR_ERR_ARG;
  if (h.method == 1) {
    memcpy(out, b + OR_HDR, (size_t)(h.g.R * h.g.C * esize_of(h.dtype)));
    return OR_OK;
  }
  int32_t *v = (int32_t *)malloc(sizeof(int32_t) * (size_t)(h.g.R * h.g.Cp));
  if (!v) return OR_ERR_NOMEM;
  rc = decode_lattice(b, &h, v);
  if (!rc)
    for (int64_t r = 0; r < h.g.R; r++) {
      float g = get_f32(b + h.o_sc + 4 * r);
      for (int64_t c = 0; c < h.g.C; c++) store_value(out, h.dtype, r * h.g.C + c, v[r * h.g.Cp + c], g);
    }
  free(v);
  return rc;
}

/* The decompression of tiles [t0, t1) only: their lattice coordinates go to
 * v_work (R x Cp int32, caller-owned) and their reconstruction to out (the
 * whole R x C container).  Calls on disjoint tile ranges touch disjoint
 * memory, so a harness may run them on several threads. */
int or_decompress_tiles(const uint8_t *b, size_t nb, int64_t t0, int64_t t1, int32_t *v_work, void *out) {
  or_header h;
  int rc = parse_header(b, nb, &h);
  if (rc) return rc;
  if (!out || !v_work || h.method != 0 || t0 < 0 || t1 > h.g.T || t0 > t1) return OR_ERR_ARG;
  rc = decode_lattice_tiles(b, &h, v_work, t0, t1);
  if (rc) return rc;
  for (int64_t t = t0; t < t1; t++)
    for (int64_t i = 0; i < h.g.tile_vecs; i++) {
      int64_t vid = tile_vector(&h.g, t, i);
      if (vid < 0) continue;
      int64_t r = vid / h.g.vpr, c0 = 8 * (vid % h.g.vpr);
      float g = get_f32(b + h.o_sc + 4 * r);
      for (int64_t c = c0; c < c0 + 8 && c < h.g.C; c++)
        store_value(out, h.dtype, r * h.g.C + c, v_work[r * h.g.Cp + c], g);
    }
  return OR_OK;
}

/* closed form: convert(f32(v * g)) for given coordinates and scales */
int or_reconstruct(const int32_t *v, const float *g, int64_t R, int64_t C, int dtype, void *out) {
  if (!v || !g || !out || R <= 0 || C <= 0) return OR_ERR_ARG;
  int64_t Cp = (C + 7) / 8 * 8;
  for (int64_t r = 0; r < R; r++)
    for (int64_t c = 0; c < C; c++) store_value(out, dtype, r * C + c, v[r * Cp + c], g[r]);
  return OR_OK;
}

/* header fields for tests: rows, cols, method, dtype, S, T, prob_bits, n_words, tile_vecs, layout, a */
int or_blob_info(const uint8_t *b, size_t nb, int64_t *i64_out, double *a_out) {
  or_header h;
  int rc = parse_header(b, nb, &h);
  if (rc) return rc;
  i64_out[0] = h.g.R;
  i64_out[1] = h.g.C;
  i64_out[2] = h.method;
  i64_out[3] = h.dtype;
  i64_out[4] = h.g.S;
  i64_out[5] = h.g.T;
  i64_out[6] = h.g.prob_bits;
  i64_out[7] = (int64_t)h.n_words;
  i64_out[8] = h.g.tile_vecs;
  i64_out[9] = h.g.layout;
  *a_out = h.a;
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Bare rANS over one symbol sequence with a single table, for pinning the   */
/* coder on its own: nstates interleaved states take symbols round-robin     */
/* (symbol k goes to state k mod nstates, in that order).                    */
/* ------------------------------------------------------------------------ */
int or_rans_encode(const uint32_t *freq, int nsym, int prob_bits, const int32_t *syms, int64_t n, int nstates,
                   uint32_t *states_out, uint16_t *words_out, int64_t *nwords_out, int64_t words_cap) {
  if (!freq || nsym <= 0 || !syms || nstates <= 0 || !states_out || !nwords_out || prob_bits < 1 || prob_bits > 11)
    return OR_ERR_ARG;
  uint32_t *cum = (uint32_t *)calloc((size_t)nsym + 1, sizeof(uint32_t));
  if (!cum) return OR_ERR_NOMEM;
  for (int s = 0; s < nsym; s++) cum[s + 1] = cum[s] + freq[s];
  if (cum[nsym] != (1u << prob_bits)) { free(cum); return OR_ERR_ARG; }
  uint32_t M = 1u << prob_bits;
  or_words rev = {0, 0, 0};
  for (int q = 0; q < nstates; q++) states_out[q] = OR_STATE_L;
  for (int64_t k = n - 1; k >= 0; k--) {
    int q = (int)(k % nstates);
    int s = syms[k];
    if (s < 0 || s >= nsym || freq[s] == 0) { free(cum); free(rev.w); return OR_ERR_ARG; }
    uint32_t f = freq[s], x = states_out[q];
    if ((uint64_t)x >= ((uint64_t)f << (OR_STATE_TOP - prob_bits))) {
      if (words_push(&rev, (uint16_t)(x & 0xffffu))) { free(cum); free(rev.w); return OR_ERR_NOMEM; }
      x >>= 16;
    }
    states_out[q] = (x / f) * M + (x % f) + cum[s];
  }
  free(cum);
  if ((int64_t)rev.n > words_cap) { free(rev.w); return OR_ERR_ARG; }
  for (uint64_t k = 0; k < rev.n; k++) words_out[k] = rev.w[rev.n - 1 - k];
  *nwords_out = (int64_t)rev.n;
  free(rev.w);
  return OR_OK;
}

int or_rans_decode(const uint32_t *freq, int nsym, int prob_bits, const uint32_t *states_in, int nstates,
                   const uint16_t *words, int64_t nwords, int64_t n, int32_t *syms_out, uint32_t *final_states) {
  if (!freq || nsym <= 0 || !states_in || nstates <= 0 || !syms_out || prob_bits < 1 || prob_bits > 11)
    return OR_ERR_ARG;
  uint32_t *cum = (uint32_t *)calloc((size_t)nsym + 1, sizeof(uint32_t));
  uint32_t *x = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)nstates);
  if (!cum || !x) { free(cum); free(x); return OR_ERR_NOMEM; }
  for (int s = 0; s < nsym; s++) cum[s + 1] = cum[s] + freq[s];
  uint32_t M = 1u << prob_bits;
  memcpy(x, states_in, sizeof(uint32_t) * (size_t)nstates);
  int64_t wp = 0;
  int rc = OR_OK;
  for (int64_t k = 0; k < n; k++) {
    int q = (int)(k % nstates);
    uint32_t slot = x[q] & (M - 1);
    int s = 0;
    while (!(cum[s] <= slot && slot < cum[s + 1])) s++;
    syms_out[k] = s;
    x[q] = freq[s] * (x[q] >> prob_bits) + slot - cum[s];
    if (x[q] < OR_STATE_L) {
      if (wp >= nwords) { rc = OR_ERR_FORMAT; break; }
      x[q] = (x[q] << 16) | words[wp++];
    }
  }
  if (rc == OR_OK && wp != nwords) rc = OR_ERR_FORMAT;
  if (final_states) memcpy(final_states, x, sizeof(uint32_t) * (size_t)nstates);
  free(cum);
  free(x);
  return rc;
}

/* frequency normalization exposed for tests */
int or_normalize(const uint64_t *cnt, int nsym, int prob_bits, uint32_t *f_out, int *nsym_out) {
  if (!cnt || nsym <= 0 || !f_out || !nsym_out) return OR_ERR_ARG;
  return normalize_counts(cnt, nsym, prob_bits, f_out, nsym_out);
}

/* model mapping exposed for tests */
int or_vector_symbols(const int32_t *v, int32_t *ctx_out, int32_t *sym_out) {
  int ctx[8];
  vector_symbols(v, ctx, sym_out);
  for (int j = 0; j < 8; j++) ctx_out[j] = ctx[j];
  return OR_OK;
}
