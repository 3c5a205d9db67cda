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
enum ep_dtype { EP_BF16 = 0, EP_FP16 = 1, EP_FP8_E4M3FN = 2, EP_INT8 = 3 };

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

/* Optional knobs for ep_compress_ex.  Zero-initialize and set what you need;
 * zero fields take the defaults. */
struct ep_options {
  double fixed_scale;  /* > 0: use this lattice resolution a, skip rate selection */
  int n_threads;       /* host encoder threads; 0 = all hardware threads */
  int reserved[6];     /* must be zero */
};

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
 * Tiles carry 64 rANS states, or 16 when the target lies below the overhead
 * of 64 (40 bits per state plus metadata; ep_blob_info reports which); the
 * README's low targets need the smaller overhead, whose streams decode about
 * 3.7x slower.
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
 * Allocates device scratch with hipMalloc for the call (about 16 KB per tile
 * of 1024 vectors, plus the word section) and frees it before returning.
 * Returns as ep_compress; EP_ERR_DEVICE if a HIP call fails, EP_ERR_NOMEM if
 * a device allocation does.
 */
int ep_compress_device(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                       const struct ep_options *opt, void *hip_stream, uint8_t **blob_out, size_t *nbytes_out);

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
  int prob_bits;     /* log2 of the frequency total */
  int64_t n_tiles;
  int64_t n_words;   /* 16-bit words in the entropy-coded section */
  double scale_a;    /* lattice resolution (row-normalized units) */
  double target_bpp; /* the target the stream was built for */
};
int ep_blob_info(const uint8_t *blob, size_t nbytes, struct ep_info *info);

/* Message for the last failing call on this thread ("" if none). */
const char *ep_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_H_ */
