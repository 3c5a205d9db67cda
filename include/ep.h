/*
 * ep.h -- C ABI of the lattice-rANS weight codec for MI355X (gfx950).
 *
 * The codec follows "EntroPack: Fast and Accurate Entropy-Coded Weight
 * Compression at Arbitrary Bitrates" (arXiv abstract on the mlsanity index
 * page): row-normalized E8 lattice quantization, a conditional probability
 * model of the lattice coordinates, resolution selection from sampled storage
 * estimates, and entropy coding in independently decodable tiles that a GPU
 * decodes and reconstructs in one fused pass.  The call surface mirrors the
 * EntroPack API reference page: compress(tensor, config) -> CompressedTensor,
 * decompress(compressed, config) -> tensor, CompressedTensor.actual_bpp and
 * storage_nbytes(include_header).
 *
 * All entry points are extern "C" and take plain pointers and sizes.  Host
 * pointers are ordinary CPU memory; "dev" pointers are device memory on the
 * current HIP device.  Every function is thread-safe; error text is kept per
 * thread (ep_last_error).
 */
#ifndef EP_H_
#define EP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Container dtypes (EntroPack README "Multiple dtypes"; the abstract lists
 * BF16, FP16, FP8 and INT8 weight containers).  FP8 is OCP E4M3FN. */
enum ep_dtype { EP_BF16 = 0, EP_FP16 = 1, EP_FP8_E4M3FN = 2, EP_INT8 = 3, EP_F32 = 4 /* ep_linear output only */ };

/* Status codes.  0 is success; a positive value is a warning with a valid
 * result; a negative value is an error and leaves outputs untouched.  The API
 * reference page ("compress") says some encoding failures warn and return an
 * uncompressed container whose method is "raw" (EP_WARN_RAW), while invalid
 * configurations and backend dispatch failures raise (negative codes). */
enum ep_status {
  EP_OK = 0,
  EP_WARN_RAW = 1,        /* stream holds the raw container bytes */
  EP_ERR_ARG = -1,        /* null pointer, bad dtype, misaligned device pointer, ... */
  EP_ERR_SHAPE = -2,      /* not 2-D or empty (rows or cols < 1), or too large */
  EP_ERR_NONFINITE = -3,  /* NaN or Inf in the input */
  EP_ERR_TARGET = -4,     /* target_bpp not finite, outside [0.001, 11] (16-bit
                             containers) or [0.001, 8) (8-bit codes), or below the
                             stream's fixed per-tile overhead for this shape */
  EP_ERR_FORMAT = -5,     /* stream header or section table is corrupt */
  EP_ERR_DEVICE = -6,     /* HIP launch or device query failed */
  EP_ERR_NOMEM = -7       /* host (or, for ep_compress_device, device) allocation failed */
};

/* Optional knobs for ep_compress_ex and ep_compress_device.  Zero-initialize
 * and set what you need; zero fields take the defaults.  Invalid values give
 * EP_ERR_ARG. */
struct ep_options {
  double fixed_scale;  /* > 0: use this lattice resolution a, skip rate selection */
  int n_threads;       /* host encoder threads; 0 = all hardware threads */
  int n_states;        /* rANS states per tile: 0 = chosen (64, or 16 when the
                          target is under 4x what 64 states cost at least),
                          16 or 64 */
  int tile_vecs;       /* E8 vectors per tile: 0 = chosen (64-state tiles: 512
                          below 2^22 vectors, else 1024; 16-state tiles: 512,
                          or 1024 for the lowest targets), 512 or 1024 */
  int sample_vecs;     /* vectors in the rate estimate's stride sample; 0 = 65536 */
  uint64_t seed;       /* phase of that sample: vector floor(k n / S) + seed mod
                          floor(n / S) for sample point k */
  int layout;          /* tile layout: EP_LAYOUT_ROWS (0) or EP_LAYOUT_BLOCKS */
  int reserved[3];     /* must be zero */
};

/* Tile layouts.  The abstract asks for independently decodable tiles and
 * leaves their shape open.
 *   EP_LAYOUT_ROWS:   tiles of 512 or 1024 E8 vectors in row-major vector
 *                     order (the default; what ep_decompress is fastest on).
 *   EP_LAYOUT_BLOCKS: each tile is the 64 x 64 weight block of rows
 *                     64 nb .. 64 nb + 63 and columns 64 kb .. 64 kb + 63
 *                     (tile nb * ceil(cols / 64) + kb; its vector i sits at
 *                     block row i / 8, block vector column i % 8; vectors
 *                     outside the matrix are absent), 64 states, 512 vectors.
 *                     This is the layout ep_linear decodes straight into a
 *                     matrix-core operand (API reference, "CompressedLinear":
 *                     reconstructed weights feed every forward call).  BF16
 *                     containers with cols % 8 == 0 only (EP_ERR_ARG /
 *                     EP_ERR_SHAPE otherwise); host encoder only
 *                     (ep_compress_device gives EP_ERR_ARG).  ep_decompress
 *                     and ep_decode_symbols read both layouts. */
enum ep_layout { EP_LAYOUT_ROWS = 0, EP_LAYOUT_BLOCKS = 1 };

/*
 * ep_compress -- lossy lattice-rANS compression of a rows x cols row-major
 * matrix (EntroPack API reference, "compress").
 *   host_src   : rows*cols elements of `dtype` (EP_BF16/EP_FP16 values,
 *                EP_FP8_E4M3FN/EP_INT8 codes), row-major, host memory.
 *   target_bpp : storage rate in bits per element, headers included; finite,
 *                non-integer allowed (README "Direct tensor compression").
 *   blob_out   : receives a malloc'ed stream; release it with ep_free.
 *   nbytes_out : receives the stream length; actual_bpp = 8*nbytes/(rows*cols).
 * Returns EP_OK, EP_WARN_RAW (lattice coding could not meet the target: the
 * stream holds the raw container), or a negative error (nothing allocated).
 * Input rules (API reference, "compress"): non-empty 2-D, finite values.
 * Rate selection runs on sampled storage estimates (plus one whole-matrix
 * histogram that codes nothing) and the stream is entropy-coded exactly once
 * (arXiv abstract: no repeated full-stream encoding).  Tiles carry 64 rANS
 * states, or 16 for low targets (ep_options; ep_blob_info reports which);
 * a state costs its symbols' information plus about 18.5 bits.  A pair of
 * states whose words exceed a count byte (only 16-state tiles at high rates)
 * is an encoding failure: EP_WARN_RAW.
 */
int ep_compress(const void *host_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                uint8_t **blob_out, size_t *nbytes_out);

/* ep_compress with options; opt may be NULL (same as ep_compress). */
int ep_compress_ex(const void *host_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                   const struct ep_options *opt, uint8_t **blob_out, size_t *nbytes_out);

/*
 * ep_compress_device -- the same compression for a matrix in device memory,
 * with the passes over its elements on the GPU (the abstract calls the
 * encoder fast and its rate selection sampled: storage estimates from a
 * sample of the vectors pick the resolution).  The stream is the one
 * ep_compress_ex returns for the same input and options, byte for byte.
 *   dev_src    : rows*cols elements of `dtype`, row-major, device memory
 *                (caller-owned, read only).
 *   opt        : as for ep_compress_ex (n_threads is not used); may be NULL.
 *   hip_stream : hipStream_t the work runs on (NULL = default stream); it is
 *                synchronized before the call returns.
 *   blob_out, nbytes_out : as for ep_compress (host memory; ep_free).
 * Allocates device scratch with hipMalloc for the call (word slots of 2 bytes
 * per element, the word section, histograms) and frees it before returning.
 * Returns as ep_compress; EP_ERR_DEVICE if a HIP call fails, EP_ERR_NOMEM if
 * a device allocation does.
 */
int ep_compress_device(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                       const struct ep_options *opt, void *hip_stream, uint8_t **blob_out, size_t *nbytes_out);

/*
 * ep_compress_device_noalloc -- ep_compress_device for callers that cannot
 * allocate memory (serving loops and harnesses that forbid hipMalloc): no
 * hipMalloc, hipFree, pinned host memory or other device allocation.  Its
 * device scratch (row sums, histograms, per-state word slots, the word
 * section) is one file-scope array of about 24 MB on each GPU the library
 * runs on, held until the process ends; the encoder's host-side tables use
 * ordinary heap memory.  The stream is the one ep_compress_device returns,
 * byte for byte, written to the caller's host buffer.
 *   dev_src, dtype, rows, cols, target_bpp, opt, hip_stream : as for
 *                ep_compress_device (the stream is synchronized before return).
 *   out        : caller-owned host buffer of `capacity` bytes for the stream.
 *                A stream whose resolution is chosen from the target never
 *                exceeds 128 + the container bytes rounded up to 16, so that
 *                capacity always suffices.
 *   nbytes_out : receives the stream length (or, with EP_ERR_ARG for a
 *                too-small buffer, the length it needs).
 * Matrices of more than 2^22 elements (rows x cols rounded up to a multiple
 * of 8) give EP_ERR_SHAPE.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents (the histograms and flags are cleared
 * before each use); overlapping calls would race on it, so the library makes
 * calls on one GPU take turns (a lock per device).
 */
int ep_compress_device_noalloc(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                               const struct ep_options *opt, void *hip_stream, uint8_t *out, size_t capacity,
                               size_t *nbytes_out);

/* Release a stream returned by ep_compress / ep_compress_ex / ep_compress_device.
 * NULL is a no-op. */
void ep_free(uint8_t *blob);

/*
 * ep_decompress -- fused GPU decode of every tile plus reconstruction of the
 * weights into the container dtype (API reference, "decompress": the result
 * has the stored shape and dtype; decoding depends only on the stored stream).
 *   host_blob, nbytes : the stream in host memory (only its header, table
 *                       and tile-offset sections are read on the host).
 *   dev_blob          : the same nbytes bytes in device memory, 16-byte aligned.
 *   dev_out           : rows*cols elements of the container dtype, row-major,
 *                       device memory, 16-byte aligned.
 *   out_dtype         : -1 or the container dtype (other conversions are not
 *                       offered).
 *   hip_stream        : hipStream_t to enqueue on (NULL = default stream).
 * Enqueues the kernel and returns; never allocates and never synchronizes.
 * Device faults surface at the caller's next synchronization.  FP8/INT8
 * containers decode to codes without the caller's row scales (API reference,
 * "CompressedFP8Linear and CompressedINT8Linear", codes()).
 */
int ep_decompress(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, void *dev_out, int out_dtype,
                  void *hip_stream);

/*
 * ep_decode_symbols -- the same fused tile decode, writing the lattice
 * coordinates v = 2*y (y the E8 point) as int16 instead of reconstructed
 * weights: rows x cols8 elements, cols8 = cols rounded up to a multiple of 8,
 * row-major, 16-byte aligned device memory.  For parity checks of the decoder
 * against an independent implementation.  Raw streams give EP_ERR_ARG.
 */
int ep_decode_symbols(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, int16_t *dev_sym,
                      void *hip_stream);

/*
 * Decode plans: ep_decompress with its host work done once per stream.  A
 * layer that keeps its weights compressed decodes them again on every forward
 * call (API reference, "CompressedLinear": reconstructed weights are used in
 * each forward call).  ep_decompress re-reads the stream's header, tables and
 * every tile offset on each call to check them and to size its launch; a plan
 * does that once, and each later decode only fills in the output pointer and
 * enqueues the kernel.
 *
 * ep_plan_create -- checks the stream exactly as ep_decompress does and
 *   records the kernel, its launch geometry and its arguments.
 *   host_blob, nbytes, dev_blob, out_dtype : as for ep_decompress; the host
 *                       stream is not read after the call returns.
 *   plan_out          : receives the plan (NULL on error).
 *   Returns EP_OK, or the error ep_decompress would return for the same
 *   stream (EP_ERR_FORMAT, EP_ERR_ARG), or EP_ERR_NOMEM.  Launches and
 *   allocates nothing on the device; the geometry is sized for the compute
 *   units of the device current at the call.
 * ep_plan_decompress -- enqueues the planned decode into dev_out (rows*cols
 *   container elements, row-major, 16-byte aligned device memory) on
 *   hip_stream (NULL = default stream).  dev_blob must still hold the same
 *   bytes and live on the stream's device.  Never allocates and never
 *   synchronizes; a plan may be used from several threads at once.
 *   EP_ERR_ARG for a NULL plan or bad dev_out, EP_ERR_DEVICE if the launch fails.
 * ep_plan_free -- releases a plan; NULL is a no-op.  The caller owns the plan
 *   and frees it once no call is using it.
 */
typedef struct ep_plan ep_plan;
int ep_plan_create(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, int out_dtype, ep_plan **plan_out);
int ep_plan_decompress(const ep_plan *plan, void *dev_out, void *hip_stream);
void ep_plan_free(ep_plan *plan);

/* actual_bpp = 8 * storage_nbytes() / (rows*cols), header included
 * (API reference, "CompressedTensor").  NaN for an invalid stream. */
double ep_actual_bpp(const uint8_t *blob, size_t nbytes);

/* storage_nbytes(include_header): the whole stream, or the stream minus its
 * fixed 128-byte header (API reference, "CompressedTensor").  -1 if invalid. */
int64_t ep_storage_nbytes(const uint8_t *blob, size_t nbytes, int include_header);

/* Stream facts for callers and tests. */
struct ep_info {
  int64_t rows, cols;
  int dtype;         /* container */
  int method;        /* 0 = lattice-rANS, 1 = raw */
  int n_states;      /* rANS states per tile */
  int tile_vecs;     /* E8 vectors per tile */
  int prob_bits;     /* log2 of the frequency total */
  int64_t n_tiles;
  int64_t n_words;   /* 16-bit words in the entropy-coded section */
  double scale_a;    /* lattice resolution (row-normalized units) */
  double target_bpp; /* the target the stream was built for */
  int layout;        /* EP_LAYOUT_ROWS or EP_LAYOUT_BLOCKS */
};
int ep_blob_info(const uint8_t *blob, size_t nbytes, struct ep_info *info);

/*
 * ep_linear -- the fused CompressedLinear product Y = X W^T with W decoded
 * on the fly (API reference, "CompressedLinear": the layer keeps its weight
 * compressed and uses the reconstructed weight in every forward call; the
 * abstract: fused symbol decoding and numerical reconstruction suit
 * Transformer prefill).  Each 64 x 64 block of W is decoded, scaled and
 * rounded to BF16 (the values ep_decompress returns) into LDS and multiplied
 * there by the BF16 matrix cores (v_mfma_f32_16x16x32_bf16), FP32
 * accumulation; W never reaches global memory.
 *   host_blob, nbytes : the stream (host copy), a lattice stream in the
 *                       blocks layout (ep_options.layout = EP_LAYOUT_BLOCKS):
 *                       W is rows x cols BF16, N = rows, K = cols.
 *   dev_blob   : the same bytes in device memory, 16-byte aligned.
 *   dev_x      : X, m x K BF16, row-major, device memory, 16-byte aligned.
 *   m          : rows of X (tokens); 0 does nothing.
 *   dev_y      : Y, m x N row-major, device memory, 4-byte aligned; dtype
 *                y_dtype: EP_F32, or EP_BF16 (FP32 sums rounded to nearest
 *                even).  Caller-owned; fully overwritten.
 *   dev_workspace, workspace_bytes : device scratch for partial sums, 16-byte
 *                aligned, caller-owned, contents ignored and overwritten; at
 *                least ep_linear_workspace_bytes(host_blob, nbytes, m) bytes
 *                lets the call split the sum over K across workgroups when
 *                the output has fewer 64-column blocks than the GPU has
 *                compute units (small m), so that every CU decodes; the
 *                partial sums are then added in a fixed order by a second
 *                kernel.  NULL or too small: no split, one workgroup per
 *                output block (the last bits may differ from a split call's;
 *                both sum in FP32 in a fixed order).
 *   hip_stream : hipStream_t the kernels are enqueued on (NULL = default).
 * Allocates nothing, does not synchronize.  The sum over K runs in a fixed
 * order for a given m and workspace (64-column blocks ascending within each
 * split, 32 columns per matrix-core step, splits added in order), so results
 * are deterministic.  Returns EP_OK; EP_ERR_ARG for a raw or row-major
 * stream, a bad y_dtype, a null or misaligned pointer; EP_ERR_SHAPE for m
 * outside [0, 2^31); EP_ERR_FORMAT for a corrupt stream; EP_ERR_DEVICE if a
 * launch fails.  Calls that share a workspace must not overlap.
 */
int ep_linear(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, const void *dev_x, int64_t m,
              void *dev_y, int y_dtype, void *dev_workspace, size_t workspace_bytes, void *hip_stream);

/* Workspace bytes ep_linear uses for m rows of X on this device (0: it does
 * not split), or a negative ep_status for a stream ep_linear refuses.  Needs
 * no GPU work; reads the device's compute-unit count. */
int64_t ep_linear_workspace_bytes(const uint8_t *host_blob, size_t nbytes, int64_t m);

/*
 * Linear plans: ep_linear with its host work done once per stream and row
 * count (the stream's header, tables and every tile offset checked, the
 * kernel, chunk size, split and grid chosen), for a layer that runs its
 * compressed weight on every forward call (API reference, "CompressedLinear").
 * ep_linear_plan_create -- as ep_linear's checks for the stream, dev_blob and
 *   m (its errors: EP_ERR_FORMAT, EP_ERR_ARG, EP_ERR_SHAPE; EP_ERR_NOMEM);
 *   plan_out receives the plan (NULL on error).  Launches and allocates
 *   nothing on the device; sized for the compute units of the current
 *   device.  The host stream is not read after the call returns.
 * ep_linear_plan_workspace_bytes -- ep_linear_workspace_bytes for the plan's
 *   stream and m (EP_ERR_ARG for a NULL plan).
 * ep_linear_plan_run -- ep_linear on the planned stream with m rows of X:
 *   dev_x, dev_y, y_dtype, dev_workspace, workspace_bytes and hip_stream as
 *   for ep_linear; dev_blob must still hold the same bytes.  Never allocates
 *   and never synchronizes; a plan may be used from several threads at once
 *   (with separate workspaces).  Results equal ep_linear's bit for bit.
 * ep_linear_plan_free -- releases a plan; NULL is a no-op.
 */
typedef struct ep_linear_plan ep_linear_plan;
int ep_linear_plan_create(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, int64_t m,
                          ep_linear_plan **plan_out);
int64_t ep_linear_plan_workspace_bytes(const ep_linear_plan *plan);
int ep_linear_plan_run(const ep_linear_plan *plan, const void *dev_x, void *dev_y, int y_dtype, void *dev_workspace,
                       size_t workspace_bytes, void *hip_stream);
void ep_linear_plan_free(ep_linear_plan *plan);

/* Message for the last failing call on this thread ("" if none). */
const char *ep_last_error(void);

/* Full entropy-coding passes the last ep_compress* call on this thread ran:
 * 1 for a lattice stream (rate selection reads sampled estimates and
 * histograms, never an encoded stream), 0 when it stopped before encoding. */
int64_t ep_last_encode_count(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_H_ */
