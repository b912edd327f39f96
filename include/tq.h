/*
 * tq.h -- C ABI of the TurboQuant KV-cache library for AMD Instinct MI355X (gfx950).
 *
 * The library compresses attention keys and values with TurboQuant and runs
 * decode attention directly on the compressed cache.  Sources of the method
 * (titles of the pages it is defined on):
 *   [Mobilint] "TurboQuant explained: near-optimal KV cache compression and why
 *              the theory breaks down in practice" (Mobilint blog);
 *   [cuTile]   function listing of DevTechJr/turboquant_cutile (codehub.bot);
 *   [tq-kv]    docs.rs page of the tq-kv crate;
 *   [ginkgoq]  "Limits And Assumptions" (ginkgoq TurboQuant docs).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  Ownership   The library never allocates device memory.  Every device buffer
 *              (rotation blob, packed cache, queries, outputs, workspace) is
 *              owned by the caller and must stay alive until the stream work
 *              that uses it has finished.  Only tq_make_rotation copies host
 *              data to the device (the layer tables, once, at set-up).
 *  Streams     `stream` is a hipStream_t passed as void* (NULL = the default
 *              stream).  Compute calls only enqueue work: results are valid in
 *              stream order, and no call synchronises except tq_make_rotation.
 *              tq_quantize_kv, tq_attn_decode and tq_dequantize enqueue kernels
 *              only (no allocation, copy or memset), so a stream capture of
 *              them replays as a HIP graph.
 *  Errors      Every argument is validated on the host before any HIP call; on
 *              an invalid argument nothing is written and nothing is enqueued.
 *              tq_last_error() returns a message for the calling thread's most
 *              recent failure.  A failed kernel launch returns TQ_ERR_HIP.
 *              No C++ exception or abort crosses this boundary.
 *  Alignment   Device pointers must be 16-byte aligned (TQ_ERR_ALIGNMENT).
 *  Threads     Calls hold no global mutable state and may be made from several
 *              threads; calls that write the same buffers must be ordered by
 *              the caller.
 *
 * Data layout in device memory
 * ----------------------------
 *  A "sequence" is one (batch, KV head) pair; a layer with B batches and Hkv
 *  KV heads has seqs = B*Hkv sequences, sequence s = b*Hkv + h.  Each holds up
 *  to `cap` tokens (cap a multiple of 8).  Per token t of sequence s the cache
 *  holds (the pages fix what is stored, not its layout; the layout below is
 *  this library's contract):
 *    idx   the b-bit codes.  A "stream" is little-endian: a b-bit code at
 *          stream position p occupies bits [p*b, p*b+b), LSB first, and bit k
 *          of a stream is bit (k mod 8) of byte k/8.
 *            keys:   one stream per token, positions = coordinates 0..d-1,
 *                    starting at byte (s*cap + t) * d*b/8;
 *            values: tokens grouped in tiles of 8; one stream per tile with
 *                    position 8*j + (t mod 8) for coordinate j (coordinate-
 *                    major tile), tile k starting at byte (s*cap/8 + k) * d*b.
 *    sign  keys with QJL: one stream of d sign bits per token (bit 1 means
 *          sign +1), starting at byte (s*cap + t) * d/8.
 *    norm  float32 ||x||_2 at index s*cap + t.
 *    rnorm keys with QJL: float32 residual norm ||r||_2 at index s*cap + t.
 *  Queries and outputs are [B][Hq][Tq][d]; query head h reads KV head
 *  h / (Hq/Hkv).  Inputs to quantize are [seqs][n][d] in the given dtype.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 2

typedef enum tq_status {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1, /* a size, count, enum or pointer is out of range */
  TQ_ERR_UNSUPPORTED = 2, /* valid in principle, not implemented (e.g. d=96) */
  TQ_ERR_ALIGNMENT = 3,   /* a device pointer is not 16-byte aligned */
  TQ_ERR_WORKSPACE = 4,   /* workspace smaller than tq_decode_workspace_bytes */
  TQ_ERR_HIP = 5          /* the HIP runtime reported an error */
} tq_status;

enum { TQ_ROT_HAAR = 0, TQ_ROT_HADAMARD = 1 };
/* Codebook laws: Lloyd-Max for N(0, 1/d), or for the exact law of a rotated
 * unit vector's coordinate, density proportional to (1 - t^2)^((d-3)/2). */
enum { TQ_LAW_GAUSSIAN = 0, TQ_LAW_BETA = 1 };
/* tq_layer.flags */
enum { TQ_LAYER_BETA_CODEBOOK = 1, TQ_LAYER_DITHER = 2, TQ_LAYER_VALUE_QJL = 4 };
enum { TQ_F32 = 0, TQ_F16 = 1 };
enum { TQ_KEYS = 0, TQ_VALUES = 1 };

/* One layer's codec: filled by tq_make_rotation, plain data, owned by the caller. */
typedef struct tq_layer {
  int32_t d;       /* head dimension: 64, 128 or 256 */
  int32_t rot;     /* TQ_ROT_HAAR or TQ_ROT_HADAMARD */
  int32_t k_bits;  /* MSE bits per key coordinate, 1..4 */
  int32_t k_qjl;   /* 1: keys also store QJL sign bits and the residual norm
                      (values do with the layer flag TQ_LAYER_VALUE_QJL) */
  int32_t v_bits;  /* MSE bits per value coordinate, 1..4 */
  int32_t flags;   /* TQ_LAYER_* bits; 0 for tq_make_rotation */
  uint64_t seed;   /* seed of the rotation, projection and sign streams */
  void* blob;      /* device: rotation, projection, signs and codebooks */
  size_t blob_bytes;
} tq_layer;

/* A compressed key or value cache for `seqs` sequences of capacity `cap`.
 * All pointers are device pointers owned by the caller. */
typedef struct tq_cache {
  uint8_t* idx;   /* codes, seqs*cap*d*bits/8 bytes */
  uint8_t* sign;  /* rows with QJL (keys with k_qjl, values with TQ_LAYER_VALUE_QJL):
                     seqs*cap*d/8 bytes; otherwise NULL */
  float* norm;    /* seqs*cap floats */
  float* rnorm;   /* rows with QJL: seqs*cap floats; otherwise NULL */
  int64_t seqs;
  int64_t cap;    /* tokens per sequence, a positive multiple of 8 */
} tq_cache;

int32_t tq_abi_version(void);
const char* tq_status_string(tq_status s);
/* Message describing the calling thread's most recent failure ("" if none). */
const char* tq_last_error(void);

/* Bytes of device memory the layer blob needs for head dimension d (0 if d is unsupported). */
size_t tq_layer_blob_bytes(int32_t d);

/* Bytes of each cache array for `which` (TQ_KEYS/TQ_VALUES): out[0]=idx,
 * out[1]=sign, out[2]=norm, out[3]=rnorm (0 where the array is not used). */
tq_status tq_cache_bytes(const tq_layer* layer, int32_t which, int64_t seqs, int64_t cap,
                         size_t out[4]);

/* Set up a layer: draws the Haar rotation Pi (QR of a seeded Gaussian with a
 * positive R diagonal; [cuTile] listing, Haar rotation function) or the randomized Hadamard H*D ([Mobilint] "How JL Matrices
 * Evolved"), the QJL projection S with i.i.d. N(0,1) entries ([Mobilint]
 * "Two-Stage Approach", stage 2), and the Lloyd-Max codebooks for the N(0,1/d)
 * coordinate law ([Mobilint] "Designing the Optimal Codebook Without Data";
 * [cuTile] listing, codebook function: both tables sorted, float32).  The random
 * matrices come from the SplitMix64 stream with Box-Muller normals, tags
 * 0 (Pi), 1 (S), 2 (D).  Builds the tables on the host in float64, copies them
 * into `dev_blob` (tq_layer_blob_bytes(d) bytes, caller-owned) on `stream` and
 * waits for the copy.  Fills *layer. */
tq_status tq_make_rotation(tq_layer* layer, int32_t d, int32_t rot, uint64_t seed,
                           int32_t k_bits, int32_t k_qjl, int32_t v_bits,
                           void* dev_blob, size_t blob_bytes, void* stream);

/* tq_make_rotation with layer options: `flags` is a combination of
 *   TQ_LAYER_BETA_CODEBOOK  key and value codebooks are the Lloyd-Max
 *                           quantizers of the exact coordinate law
 *                           f(t) ~ (1 - t^2)^((d-3)/2) on [-1, 1] ([Mobilint]
 *                           "Coordinates Become Predictable After Rotation" and
 *                           "Designing the Optimal Codebook Without Data": the
 *                           integrals done numerically) instead of N(0, 1/d).
 *   TQ_LAYER_DITHER         dithered randomized-Hadamard variant
 *                           (thelatestinai.com paper page 2606.10458, third
 *                           abstract: HD, then a random scalar offset
 *                           subtracted before quantizing): each token's
 *                           rotated coordinates are coded as
 *                           #{i : beta_i < y_j - delta} and reconstructed as
 *                           c[idx] + delta, delta = w (u - 1/2) with w the
 *                           spacing of the codebook's two central centroids
 *                           and u the uniform of output seq * 2^32 + t + 1 of
 *                           the layer's SplitMix64 stream with tag 3 (keys) or
 *                           4 (values), regenerated wherever it is needed.
 *                           Needs rot = TQ_ROT_HADAMARD and k_qjl = 0.
 *   TQ_LAYER_VALUE_QJL      values carry QJL too (TurboQuant_prod on V:
 *                           [Mobilint] "Two-Stage Approach", applied to the
 *                           value rows): value caches then hold sign
 *                           (d/8 bytes per token, one stream per token as for
 *                           keys) and rnorm, and every value enters decode as
 *                           its two-stage reconstruction
 *                           n (R^T c[idx] + sqrt(pi/2)/d gamma S^T sigma).
 *                           Such layers run the reference (scalar) quantize
 *                           and decode kernels.  Not with TQ_LAYER_DITHER.
 * Unknown flag bits, TQ_LAYER_DITHER without those, or both DITHER and
 * VALUE_QJL, give TQ_ERR_INVALID_ARG. */
tq_status tq_make_layer(tq_layer* layer, int32_t d, int32_t rot, uint64_t seed, int32_t k_bits,
                        int32_t k_qjl, int32_t v_bits, int32_t flags, void* dev_blob, size_t blob_bytes,
                        void* stream);

/* Host-only: the float64 rotation matrix R (Pi or H*D, row-major, y = R u) and
 * projection S (row-major) the layer with this (d, rot, seed) uses.  Either
 * output may be NULL.  No GPU needed. */
tq_status tq_host_tables(int32_t d, int32_t rot, uint64_t seed, double* rotation,
                         double* projection);

/* Host-only: the float32 codebook for `bits` at head dimension d: 2^bits sorted
 * centroids and 2^bits-1 sorted boundaries ([cuTile] codebook function). */
tq_status tq_get_codebook(int32_t d, int32_t bits, float* centroids, float* boundaries);

/* Host-only: tq_get_codebook for a codebook law (TQ_LAW_GAUSSIAN or TQ_LAW_BETA). */
tq_status tq_get_codebook_law(int32_t d, int32_t bits, int32_t law, float* centroids, float* boundaries);

/* Compress tokens t0..t0+n-1 of every sequence into `cache` ([cuTile] listing,
 * key and value compression functions, values without QJL; [Mobilint]
 * "Two-Stage Approach").  Per token: store n = ||x||; rotate
 * u = x/n (u = 0 when n = 0); code each coordinate as #{i : beta_i < y_j};
 * bit-pack.  Keys with QJL also store gamma = ||r|| and sign(S r) for the
 * residual r = u - R^T c[idx] (sign(0) = +1).  x is [seqs][n][d] of `dtype`
 * (TQ_F32 or TQ_F16), device memory.  Tokens outside [t0, t0+n) are left as
 * they were, including the other tokens that share a value tile. */
tq_status tq_quantize_kv(const tq_layer* layer, int32_t which, const void* x, int32_t dtype,
                         int64_t seqs, int64_t n, int64_t t0, const tq_cache* cache,
                         void* stream);

/* Workspace bytes tq_attn_decode needs for this shape. */
size_t tq_decode_workspace_bytes(const tq_layer* layer, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t Tq, int64_t N);

/* Decode attention on the compressed cache ([cuTile] listing,
 * asymmetric score estimator, the attention pipeline and the fused attention
 * function with online softmax and values decoded on chip; [Mobilint] "Two-Stage Approach": <q, x~> = <Pi q, y~>).  For each
 * query row the query is rotated once (R q, S q); key t scores
 *   s_t = n_t * (<R q, c_k[idx_t]> + gamma_t*sqrt(pi/2)/d * <S q, sigma_t>) / sqrt(d);
 * softmax over keys 0..N-1 (with `causal`, query i of Tq sees keys
 * t <= N - Tq + i); the values n_v * c_v[idx_v] are summed in the rotated
 * domain and the sum is un-rotated once per query row.
 * q: [B][Hq][Tq][d] of q_dtype; out: [B][Hq][Tq][d] float32; scores: NULL or
 * [B][Hq][Tq][N] float32 (masked keys get -inf).  K and V hold B*Hkv
 * sequences with at least N tokens.  `workspace`: device scratch of at least
 * tq_decode_workspace_bytes(...) bytes, 256-byte aligned. */
tq_status tq_attn_decode(const tq_layer* layer, const void* q, int32_t q_dtype, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t Tq, int64_t N, int32_t causal,
                         const tq_cache* K, const tq_cache* V, float* out, float* scores,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Maximum decode scratch of tq_attn_decode_static (bytes). */
#define TQ_DECODE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

/* tq_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * tq_attn_decode; the split partials go to a fixed 16 MiB device array of the
 * library instead (TQ_DECODE_STATIC_SCRATCH_BYTES; each GPU the library runs
 * on holds its own copy until the process ends).  A shape whose
 * tq_decode_workspace_bytes exceeds that returns TQ_ERR_WORKSPACE with nothing
 * enqueued.  The first call on a device looks up that device's copy (a host
 * call, no allocation); no call allocates or frees memory.  Nothing in the
 * array needs to start at zero: every split writes its partial row before the
 * merge reads it.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents, so calls that overlap on one GPU (concurrent
 * streams, threads) race: the caller must order them. */
tq_status tq_attn_decode_static(const tq_layer* layer, const void* q, int32_t q_dtype, int32_t B,
                                int32_t Hq, int32_t Hkv, int32_t Tq, int64_t N, int32_t causal,
                                const tq_cache* K, const tq_cache* V, float* out, float* scores,
                                void* stream);

/* Reconstruct tokens 0..n-1 of every sequence: x_hat = n * R^T c[idx]
 * ([cuTile] listing, decompression function).  out is
 * [seqs][n][d] of out_dtype (TQ_F32 or TQ_F16). */
tq_status tq_dequantize(const tq_layer* layer, int32_t which, const tq_cache* cache, int64_t n,
                        void* out, int32_t out_dtype, void* stream);

/* Two-stage reconstruction of rows with QJL ([Mobilint] "Two-Stage Approach",
 * final reconstruction): tokens 0..n-1 of every sequence become
 *   x_hat = n * (R^T c[idx] + sqrt(pi/2)/d * gamma * S^T sigma),
 * the MSE reconstruction of tq_dequantize plus the QJL back-projection of the
 * residual's sign bits.  Same arguments as tq_dequantize; `which` must be
 * TQ_KEYS of a layer with k_qjl = 1, or TQ_VALUES of a layer with
 * TQ_LAYER_VALUE_QJL, and the cache must hold sign and rnorm (else
 * TQ_ERR_INVALID_ARG).  Keys of a Haar layer at d = 64 or 128: one launch on
 * `stream` that stores each row once.  Otherwise two: the MSE rows, then the
 * QJL term added to them in place. */
tq_status tq_dequantize_prod(const tq_layer* layer, int32_t which, const tq_cache* cache, int64_t n,
                             void* out, int32_t out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
