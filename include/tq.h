/*
 * tq.h -- C ABI of libtq: SRHT KV-cache compression and decode attention over
 * the packed cache, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are the pages' titles and sections):
 *  - Encode: each 128-dim head vector x of a key or value is rotated by the
 *    randomized Walsh-Hadamard transform R = D H D / sqrt(d) ("TurboQuant-MLX
 *    v2.0", What's New > Walsh-Hadamard Rotation; How It Works > Pipeline),
 *    its L2 norm n is stored, and every coordinate of u = sqrt(d) R x / n is
 *    scalar-quantised against a Lloyd-Max Gaussian codebook or a symmetric
 *    uniform grid ("TurboMOQ", Architecture) at a per-page bit width of 1-8
 *    ("TurboMOQ", Architecture: per-head adaptive bit width), then bit-packed.
 *    Keys may carry a 1-bit QJL residual sign sketch with a per-vector scale
 *    ("TurboMOQ", QJL residual correction; "TurboQuant-MLX v2.0", Pipeline).
 *  - Decode attention: one query per session attends over every cached token:
 *    softmax(q . k / sqrt(d)) . v, reading packed pages directly (scores in the
 *    rotated domain, value accumulation in the rotated domain and one inverse
 *    rotation at the end, which factors the Walsh-Hadamard transform out of the
 *    V accumulation as the MLX TurboQuant skill page describes for its Metal
 *    kernels, Path A > Optimisations Metal) and fp16 pages
 *    for the attention sink and other uncompressed tokens ("TurboQuant-MLX
 *    v2.0", What's New > FP16 Attention Sinks).
 *
 * Conventions shared by every call:
 *  - head_dim d = 128, page = 64 tokens of one (session, KV head), JL dim m = 128.
 *  - Device pointers are HIP device addresses owned by the caller.  The library
 *    never allocates, frees or synchronises device memory; calls that take a
 *    stream enqueue work on it (a hipStream_t passed as void*; NULL = default
 *    stream) and return after the enqueue.
 *  - Every call validates its arguments on the host before any HIP call; on a
 *    validation failure it returns a negative status, writes nothing and
 *    records a message readable with tq_last_error() (per thread).
 *  - TQ_ERR_DEVICE reports a failed kernel launch (hipGetLastError after the
 *    launch); faults during execution surface at the caller's next
 *    synchronisation, as for any HIP kernel.
 *
 * Rotation: R = D H D / sqrt(d), H the Sylvester Hadamard matrix in natural
 * order, D = diag(+-1) from the layer's sign mask.  R is symmetric and its own
 * inverse.
 *
 * Quantisation: code_j = #{k : t_k <= u_j} over the ascending float32
 * boundaries t of the page's bit width (ties round up; code 0 is the most
 * negative centroid).  Dequantisation: xhat = (n / sqrt(d)) R c[code].
 *
 * QJL (keys): r = x - xhat, z_i = [(S r)_i >= 0], gamma = ||r||;
 * rhat = sqrt(pi/2)/m * gamma * S^T (2z - 1); the attended key is xhat + rhat.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1, /* null pointer, bad size/range/kind             */
  TQ_ERR_UNSUPPORTED = -2, /* head_dim != 128, bits outside 1..8, jl != 128, GQA group not 1/2/4/8 */
  TQ_ERR_ALIGNMENT = -3,   /* pointer or stride not 16-byte aligned          */
  TQ_ERR_WORKSPACE = -4,   /* workspace smaller than tq_decode_workspace_bytes */
  TQ_ERR_DEVICE = -5       /* HIP reported an error when launching           */
};

enum { TQ_CODEBOOK_LLOYD_MAX = 0, TQ_CODEBOOK_UNIFORM = 1, TQ_CODEBOOK_BETA = 2,
       TQ_CODEBOOK_FITTED = 3 /* a table from tq_calibrated_table */,
       TQ_CODEBOOK_POLAR = 4 /* PolarQuant, see tq_build_codebook */ };
enum { TQ_DTYPE_F32 = 0, TQ_DTYPE_F16 = 1 };
enum { TQ_QJL_SCORE_UNBIASED = 0, TQ_QJL_SCORE_SIGN = 1 };

#define TQ_HEAD_DIM 128
#define TQ_PAGE_TOKENS 64
#define TQ_JL_DIM 128
/* floats in one codebook table (all bit widths of one kind), see tq_codebook_table */
#define TQ_CODEBOOK_TABLE_FLOATS 12288

/* ------------------------------------------------------- page descriptors
 * A cache is a caller-owned byte pool plus a page table of uint64
 * descriptors, one per (session, KV head, page):
 *   bits  0..47  byte offset of the page in the pool (multiple of 256)
 *   bits 48..51  k_bits (1..8); 0 marks an fp16 page
 *   bits 52..55  v_bits (1..8); 0 for an fp16 page
 *   bit  56      the page carries a QJL residual for its keys
 *   bit  57      pending: the page is still filling and is stored as an fp16
 *                page (a 32 KiB slot) until tq_append_kv writes its 64th token
 *                and encodes it in place into the packed format the other
 *                bits name ("TurboQuant-MLX v2.0", What's New > Dynamic Chunk
 *                Buffering: tokens are buffered until a chunk is complete)
 *   bit  63      present
 * Packed page layout (bytes, in order):
 *   K codes   1024*k_bits : 64 streams of 128 codes; stream t = token t's
 *             codes of coordinates 0..127; a stream is its codes LSB-first
 *             (code n at bits n*b..n*b+b-1), i.e. b little-endian 128-bit
 *             words, and word w of stream s is at byte (w*64 + s)*16.
 *   K norms   64 x float32
 *   [QJL]     64 x 16 B sign words (bit i of token t's word = z_i), then
 *             64 x float32 gamma
 *   V codes   1024*v_bits : 64 streams as above, but stream s = n + 32P
 *             (n < 32, P in {0, 1}) holds one coordinate pair over the
 *             page: token t's codes of coordinates c0 and c0 + 1 at stream
 *             positions 2t and 2t+1, where c0 = 64*((n >> 2) & 1) + 32P +
 *             8*(n >> 3) + 2*(n & 3)
 *   V norms   64 x float32
 * fp16 page: 64 rows of K then 64 rows of V, fp16, 128 values per row.
 * These layouts are a convention of this library (the pages name bit packing
 * only as a utility module); tq_page_bytes() gives the sizes.              */
#define TQ_PAGE_PRESENT (1ull << 63)
#define TQ_CACHE_COMMON_PAGES 1
#define TQ_CACHE_OTHER_PAGES 2
#define TQ_CACHE_WIDE_PAGES 4
#define TQ_PAGE_QJL (1ull << 56)
#define TQ_PAGE_PENDING (1ull << 57)
#define TQ_PAGE_OFFSET_MASK ((1ull << 48) - 1)
#define TQ_RETIER_FROM_PACKED 1
#define TQ_RETIER_FROM_FP16 2

/* Bytes of one page: k_bits = 0 (and v_bits = 0, qjl = 0) for an fp16 page.
 * Returns 0 for an invalid combination. */
size_t tq_page_bytes(int k_bits, int v_bits, int qjl);

/* Builds a page descriptor; returns 0 for an invalid combination or an offset
 * that is not a multiple of 256 or does not fit 48 bits. */
uint64_t tq_page_descriptor(uint64_t offset, int k_bits, int v_bits, int qjl);

/* ------------------------------------------------------------ descriptors */
typedef struct tq_layer {
  int32_t head_dim;          /* must be 128                                      */
  int32_t k_codebook;        /* TQ_CODEBOOK_* used by every packed K block       */
  int32_t v_codebook;        /* TQ_CODEBOOK_* used by every packed V block       */
  int32_t jl_dim;            /* 128; read only by pages with the QJL bit         */
  const uint32_t* sign_mask; /* device, 4 words: bit j set <=> D_j = -1          */
  const float* k_table;      /* device, TQ_CODEBOOK_TABLE_FLOATS floats from
                                tq_codebook_table(k_codebook)                    */
  const float* v_table;      /* device, same for v_codebook                      */
  const float* qjl_s;        /* device, S as 128 x 128 float32 row-major, or
                                NULL when no page of the cache uses QJL          */
} tq_layer;

typedef struct tq_cache {
  int32_t n_sessions;        /* B                                                */
  int32_t n_kv_heads;        /* H_kv                                             */
  int32_t max_pages;         /* row length of the page table                     */
  int32_t page_classes;      /* which page classes the table holds, as the host
                                that built it knows: TQ_CACHE_COMMON_PAGES (a
                                1-4 bit K and V page without QJL) |
                                TQ_CACHE_WIDE_PAGES (5-8 bit K and V, no QJL) |
                                TQ_CACHE_OTHER_PAGES (fp16, QJL or mixed
                                widths; a pending page counts here and in the
                                class of its packed format); decode attention
                                skips the work of a class whose bit is clear.
                                0 = unknown (all run).  A set that leaves out a
                                class present in the table makes decode ignore
                                those pages.                                     */
  const int32_t* n_tokens;   /* device [B]: tokens cached per session; decode
                                attends to tokens [0, n_tokens[b]) and needs
                                n_tokens[b] <= 64 * max_pages                    */
  const uint64_t* pages;     /* device [B][H_kv][max_pages] descriptors          */
  void* pool;                /* device byte pool, 256-byte aligned               */
  uint64_t pool_bytes;       /* pool size; pages outside it are never touched    */
  const uint8_t* unit_classes; /* host [B][H_kv] or NULL: the page classes each
                                (session, KV head) holds, in the bits of
                                page_classes.  Decode attention then launches a
                                class's workgroups only for the units whose bit
                                is set (and that page_classes admits), so a
                                class held by a few heads costs no workgroups
                                on the others; a unit whose bit is clear has its
                                pages of that class ignored, as with
                                page_classes.  Read on the host during the call
                                only (a captured graph keeps the lists of its
                                capture).  NULL, or more than
                                TQ_MAX_LISTED_UNITS units, launches every unit
                                of every admitted class.                        */
} tq_cache;

#define TQ_MAX_LISTED_UNITS 512

typedef struct tq_kv_input {
  const void* k;             /* device: element (b, h, t, j) of the call's keys at
                                k + ((b*stride_b + h*stride_h + t*stride_t) + j)
                                elements, t = 0..ntok-1 for cache token tok0+t   */
  const void* v;             /* device, same shape and strides as k              */
  int32_t dtype;             /* TQ_DTYPE_F16 or TQ_DTYPE_F32                     */
  int32_t tok0;              /* first cache token written; multiple of 64        */
  int32_t ntok;              /* tokens in this call (>= 1)                       */
  int32_t reserved;          /* 0                                                */
  int64_t stride_b, stride_h, stride_t;  /* in elements; rows 16-byte aligned   */
  int32_t* error_flags;      /* device int or NULL: kernels OR in
                                1 = a packed page only partly covered by the call
                                    (left untouched),
                                2 = a page descriptor in range not present,
                                4 = a page outside the pool (left untouched)     */
} tq_kv_input;

typedef struct tq_token_input {
  const void* k;             /* device: element (b, h, j) of the new keys at
                                k + (b*stride_b + h*stride_h + j) elements       */
  const void* v;             /* device, same shape and strides as k              */
  int32_t dtype;             /* TQ_DTYPE_F16 or TQ_DTYPE_F32 (rounded to fp16)   */
  int32_t reserved;          /* 0                                                */
  int64_t stride_b, stride_h;  /* in elements; rows 16-byte aligned             */
  int32_t* error_flags;      /* device int or NULL: kernels OR in
                                2 = the page at the position is not present,
                                4 = the page is outside the pool or its pending
                                    format is invalid (left untouched),
                                16 = the position is past the page table,
                                32 = the page at the position is already packed */
} tq_token_input;

typedef struct tq_query {
  const void* q;             /* device: element (b, h, j) at
                                q + b*stride_b + h*stride_h + j elements         */
  int32_t dtype;             /* TQ_DTYPE_F16 or TQ_DTYPE_F32                     */
  int32_t n_q_heads;         /* H_q = G * H_kv, G in {1, 2, 4, 8}; query head h
                                reads KV head h / G                              */
  int64_t stride_b, stride_h;
  float softmax_scale;       /* 0 selects 1/sqrt(128)                            */
  int32_t qjl_scoring;       /* how pages with a QJL sketch score it:
                                TQ_QJL_SCORE_UNBIASED (0): gamma sqrt(pi/2)/m
                                  z . (S q), the estimator of q . r;
                                TQ_QJL_SCORE_SIGN (1): gamma (pi/2)/m ||q||
                                  z . sign(S q), the sign-agreement form
                                ("TurboQuant-MLX v2.0", RaBitQ vs QJL
                                correction and Implementation Status: both
                                sides as signs, scaled by pi/2), which
                                estimates ||q|| ||r|| asin(cos(q, r))        */
} tq_query;

/* --------------------------------------------------------- host-only calls */

/* Codebook for one bit width ("TurboMOQ", Architecture: Lloyd-Max codebook;
 * Limitations: without calibration data the method uses a symmetric grid).
 * kind = TQ_CODEBOOK_LLOYD_MAX: the MSE-optimal 2^bits-level quantiser of
 *   N(0,1) (the unique fixed point of the centroid and midpoint conditions);
 * kind = TQ_CODEBOOK_UNIFORM: levels (k - (L-1)/2) * delta with the
 *   MSE-optimal delta for N(0,1), boundaries at midpoints;
 * kind = TQ_CODEBOOK_BETA: the MSE-optimal quantiser of one coordinate of
 *   sqrt(128) times a uniformly random unit vector of R^128 (density
 *   proportional to (1 - u^2/128)^(125/2); u^2/128 ~ Beta(1/2, 127/2)), the
 *   exact law of a rotated, normalised coordinate when the direction is random
 *   ("TurboMOQ", Head-to-Head Comparison and Project Structure: Beta-CDF,
 *   Beta-distribution codebooks);
 * kind = TQ_CODEBOOK_POLAR: PolarQuant ("TurboQuant-MLX v2.0", How It Works >
 *   Pipeline: each rotated coordinate pair as a radius and an angle, quantised
 *   independently).  A part coded at width b holds, for pair i, the radius code
 *   at stream position 2i and the angle code at 2i+1, so a polar page has the
 *   scalar layout and size.  This call gives the radius quantiser: the 2^bits
 *   Lloyd-Max levels of Rayleigh(1) (the radius of a standard 2-D Gaussian
 *   pair) and their midpoints.  The angle theta = atan2(u_2i+1, u_2i) takes
 *   sector floor((theta + pi) 2^bits / (2 pi)) mod 2^bits, reconstructed at the
 *   sector's middle.  Widths 1..4 only (pages of a polar part wider than 4
 *   bits are refused by the kernels).
 * Writes 2^bits ascending centroids and 2^bits - 1 boundaries (caller-owned
 * host arrays), each the float32 nearest the exact value.  Pure, deterministic
 * and thread-safe; bits in 1..8. */
int tq_build_codebook(int bits, int kind, float* centroids, float* boundaries);

/* The table kernels read, for every bits = 1..8: the centroids at float offset
 * 2^bits - 2 and the boundaries at 510 + 2^bits - bits - 1; then, for the
 * encoder, a lookup grid per width (header {S, O, n_bins, offset} at
 * 1024 + 4 (bits - 1); pair tables of widths 1..4 at float offset 1056 (width
 * b at float2 entry 0, 4, 20, 84 for b = 1, 2, 3, 4; entry lo | hi << b holds
 * the two values of a coordinate pair coded (lo, hi): (c[lo], c[hi]) for a
 * scalar codebook, radius level lo in sector hi's middle direction for
 * PolarQuant); the grids' n_bins entries {count of boundaries below the bin
 * (u32), the one boundary inside the bin widened by a quarter bin each side
 * (f32, or 3e38)} at `offset`), so that code(u) = count + [u >= boundary] at
 * bin floor(u S + O) clamped to [0, n_bins); a grid of n_bins = 256 is instead
 * indexed by u S + O rounded to the nearest integer (ties to even) and
 * saturated to [0, 255].  The tail is zero.  Writes
 * TQ_CODEBOOK_TABLE_FLOATS floats to a host array (copy it to the device for
 * tq_layer). */
int tq_codebook_table(int kind, float* table);

/* The table of a PolarQuant part whose radius and angle take widths of their
 * own ("TurboQuant-MLX v2.0", Quick Start: r_bits and theta_bits are separate;
 * "turboquant-mlx" README, apply_turboquant_cache: k/v_theta_bits,
 * k/v_radius_bits).  A page of width b keeps the scalar layout and size (2b
 * bits per coordinate pair); angle_shift t (-3..3) gives the radius r = b - t
 * bits (the Lloyd-Max levels of Rayleigh(1) at r bits) and the angle a = b + t
 * bits (2^a sectors), and the pair field F = radius code | angle code << r is
 * stored as two b-bit codes, F's low b bits at stream position 2i and its high
 * b bits at 2i + 1.  The pair table of width b is indexed by F; the shift is
 * kept in the table's last entry, where the encoders read it.  Use with
 * k_codebook / v_codebook = TQ_CODEBOOK_POLAR; tq_codebook_table(POLAR) is
 * shift 0.  Pages wider than 4 bits, or whose width cannot carry the shift
 * (r or a below 1), are refused by the encoders (error flag 4) and must not be
 * decoded.  TQ_ERR_UNSUPPORTED for a shift outside -3..3. */
int tq_polar_table(int angle_shift, float* table);

/* Codebook fitted to sample head vectors ("TurboMOQ", Quick Start: calibrate
 * codebooks from sample data; Architecture: Lloyd-Max codebook (k-means);
 * Limitations: Lloyd-Max codebooks need sample data).  The samples are the
 * rotated, normalised coordinates u = sqrt(128) R x / ||x|| of the n nonzero
 * vectors (host float32, n x 128, rotated with the layer's signs) together
 * with their mirror images -u, so the codebook is symmetric as the encoder
 * requires.  Lloyd's iteration (k-means in one dimension): levels start at the
 * Gaussian Lloyd-Max ones; each sweep assigns every sample to the cell between
 * the midpoints of neighbouring levels and moves each level to its cell's mean
 * (a level whose cell is empty stays), until no sample changes cell or 200
 * sweeps.  Writes 2^bits ascending centroids and their 2^bits - 1 midpoints
 * (float32 of the double values).  Deterministic; host memory only. */
int tq_fit_codebook(const float* vectors, size_t n, const int8_t* signs, int bits,
                    float* centroids, float* boundaries);

/* A codebook table (as tq_codebook_table writes) of the codebooks
 * tq_fit_codebook fits at every width 1..8 from the same samples; use it as
 * tq_layer.k_table or v_table with kind TQ_CODEBOOK_FITTED.
 * TQ_ERR_UNSUPPORTED when a width's boundaries are too close together for the
 * encoder's lookup grid (too few distinct samples). */
int tq_calibrated_table(const float* vectors, size_t n, const int8_t* signs, float* table);

/* Layer randomness from a seed ("TurboQuant-MLX v2.0", What's New: seed 42;
 * MLX TurboQuant skill page, Standalone Benchmark: one cache per layer seeded
 * 42 + layer).  Stream = counter-based SplitMix64 seeded with seed + layer.
 * Outputs 1..head_dim give signs[j] = -1 if the top bit is set, else +1; when
 * qjl_s is not NULL the following outputs, as uniforms (z >> 11) * 2^-53
 * taken in pairs through Box-Muller (cos then sin), fill S (jl_dim x
 * head_dim, row-major float32).  Host arrays; head_dim = jl_dim = 128. */
int tq_layer_params(uint64_t seed, int layer, int head_dim, int jl_dim,
                    int8_t* signs, float* qjl_s);

/* Packs 128 signs (+1 / -1) into the 4-word mask tq_layer.sign_mask expects. */
int tq_sign_mask(const int8_t* signs, int head_dim, uint32_t* mask);

/* Workspace tq_decode_attention needs for this cache and query-head count. */
size_t tq_decode_workspace_bytes(const tq_cache* cache, int n_q_heads);

/* Bytes of a cache: the sum of tq_page_bytes over the given descriptors
 * (a host copy of the page table, n entries; absent pages count zero, pending
 * pages count as fp16 pages). */
size_t tq_cache_bytes(const uint64_t* host_pages, size_t n);

const char* tq_status_string(int status);
const char* tq_last_error(void);

/* The device checks of a checked build (the library compiled with
 * TQ_DEVICE_CHECKS=1, libtq_checked.so): the kernels verify their index
 * invariants as they run, record a violated one as a bit, and clamp the index
 * so that the access stays in bounds.  *flags receives the bits recorded since
 * the last reset (1 encode lookup grid, 2 encode streams and code rows, 4 QJL
 * key encoder LDS, 8 decode tables and weight rows, 16 decode descriptor and
 * partial slots, 32 combine lists, 64 append and re-tier); reset != 0 clears
 * them.  Synchronous: waits for the device's work.  A release build sets
 * *flags = 0 and returns TQ_ERR_UNSUPPORTED; TQ_ERR_INVALID_ARG for a null
 * flags. */
int tq_device_checks(uint32_t* flags, int reset);

/* ----------------------------------------------------------- device calls */

/* Encodes tokens [tok0, tok0 + ntok) of every (session, KV head) into the
 * pages the page table names ("TurboQuant-MLX v2.0", What's New > Dynamic
 * Chunk Buffering: compression fires on whole 64-token chunks).  A packed
 * page is written only when the call covers all 64 of its tokens; an fp16
 * page receives the covered rows (rounded to fp16 when the input is fp32).
 * Pages are independent: calls over disjoint token ranges may be issued in any
 * order.  Keys of QJL pages also get their sign sketch and gamma. */
int tq_encode_kv(const tq_layer* layer, const tq_cache* cache,
                 const tq_kv_input* in, void* stream);

/* tq_encode_kv with its launch shape chosen by the caller, for checking that
 * the result does not depend on it (the kernels' LDS reuse and barriers):
 * pages_per_block = pages each workgroup of the bulk encoder takes in turn
 * (1..16, 0 = the default 4), qjl_workgroups = the persistent workgroups of
 * the QJL key encoder (0 = one per compute unit; more than the work needs are
 * not launched).  The pages written are byte-identical for every shape.
 * TQ_ERR_INVALID_ARG for a shape outside those ranges, else as tq_encode_kv. */
int tq_encode_kv_shaped(const tq_layer* layer, const tq_cache* cache,
                        const tq_kv_input* in, int pages_per_block,
                        int qjl_workgroups, void* stream);

/* One step of a decode loop ("TurboQuant-MLX v2.0", What's New > FP16
 * Attention Sinks and Dynamic Chunk Buffering: recent tokens stay fp16 until a
 * 64-token chunk is complete, then the chunk is compressed).  For every
 * session b and KV head h, writes the new key and value rows (fp16) as token
 * n_tokens[b] of the cache: row n_tokens[b] mod 64 of the page that holds it,
 * which must be an fp16 page or a pending page.  A pending page that receives
 * its 64th token is encoded in place (same slot) into the packed format its
 * descriptor names, exactly as tq_encode_kv would encode those 64 fp16 rows,
 * and its pending bit is cleared.  Then n_tokens[b] += 1 for every session.
 * Writes the pool, the page table (pending bits) and n_tokens, which must be
 * device memory the call may modify.  Errors found on the device are OR-ed
 * into in->error_flags; n_tokens advances regardless. */
int tq_append_kv(const tq_layer* layer, const tq_cache* cache, const tq_token_input* in,
                 void* stream);

/* Re-tiers pages in place ("TurboMOQ", Progressive temporal tiering: older
 * chunks move from fp16 to 4/4, 3/2 and 2/1 bits; Attention-weighted tier
 * demotion: the tier of a chunk may also follow the attention it receives).
 * For i in [0, n): the page at flat page-table position page_index[i]
 * (= (b * n_kv_heads + h) * max_pages + p) takes descriptor new_desc[i], a
 * present packed format (not pending):
 *   - from an fp16 page: its 64 fp16 rows are encoded into the new format
 *     (QJL allowed), exactly as tq_encode_kv would encode them;
 *   - from a packed page without QJL: to k_bits' <= k_bits and
 *     v_bits' <= v_bits without QJL, each code c of width b becomes the
 *     width-b' code of centroid c_b[c] (the count of width-b' boundaries at
 *     or below it) and the norms are kept: rotation and norm are unchanged,
 *     so the page is re-coded without being decoded.
 * The new slot (offset of new_desc[i]) is the old one or a range that does
 * not overlap it; slots of different listed pages must not overlap, and
 * no position may be listed twice.  page_index and new_desc are device
 * arrays (8-byte aligned) of n entries; the call writes the pool and the page
 * table.  Decode after the call needs tq_cache.page_classes to cover the new
 * formats.  sources says which source kinds the list holds, as the caller
 * knows: TQ_RETIER_FROM_PACKED | TQ_RETIER_FROM_FP16, 0 = unknown (both); the
 * work of a kind left out is not launched, and a listed page of that kind is
 * refused (flag 64).  Errors found on the device are OR-ed into error_flags
 * (device int or NULL), and the page is left untouched:
 *   2 = the old or new descriptor is not present,
 *   4 = invalid format, a slot outside the pool, or overlapping old and new
 *       slots,
 *   8 = a QJL target and layer->qjl_s is NULL,
 *   16 = page_index[i] outside the page table,
 *   64 = an unsupported change: a pending page, a QJL page as the source or
 *       (from a packed page) as the target, a packed width that grows, or a
 *       source kind that `sources` leaves out.  */
int tq_retier_pages(const tq_layer* layer, const tq_cache* cache, const int64_t* page_index,
                    const uint64_t* new_desc, int n, int sources, int32_t* error_flags,
                    void* stream);

/* out[b][h][0..127] (device float32, row stride 128, B x H_q rows) =
 * softmax_t(scale * q_bh . k_t) . v_t over t in [0, n_tokens[b]), where k_t,
 * v_t are the fp16 values of fp16 pages and the dequantised vectors (keys plus
 * the QJL residual where present) of packed pages.  Needs a device workspace of
 * tq_decode_workspace_bytes(cache, n_q_heads) bytes (16-byte aligned; contents
 * on entry are ignored).  Launches three kernels on the stream: query
 * rotation, split-K over pages, and the combine. */
int tq_decode_attention(const tq_layer* layer, const tq_cache* cache,
                        const tq_query* query, float* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* tq_decode_attention, also returning the attention mass of every page
 * ("TurboMOQ", Attention-weighted tier demotion: a policy reassigns tiers from
 * the attention weights of each decode step, and pins what stays important).
 * page_mass[b][hq][p] (device float32, B x H_q x max_pages, contiguous, 4-byte
 * aligned; every entry is written) = the sum over the tokens t < n_tokens[b]
 * held by page p of the softmax weight query head hq gives t; 0 for pages
 * past n_tokens[b] or that decode skips (absent, outside the pool, or of a
 * class page_classes leaves out).  A row's masses sum to 1 up to rounding.
 * Same workspace and errors as tq_decode_attention, plus TQ_ERR_INVALID_ARG
 * for a null page_mass. */
int tq_decode_attention_mass(const tq_layer* layer, const tq_cache* cache,
                             const tq_query* query, float* out, float* page_mass,
                             void* workspace, size_t workspace_bytes, void* stream);

/* tq_decode_attention, also returning the attention weight of every token
 * ("TurboMOQ", Attention-weighted tier demotion: the policy tracks importance
 * per position, {position: tier}).  token_mass[b][hq][t] (device float32,
 * B x H_q x (max_pages x 64), contiguous, 16-byte aligned; every entry is
 * written) = the softmax weight query head hq gives token t of session b; 0
 * for t >= n_tokens[b] and for the tokens of pages decode skips (absent,
 * outside the pool, or of a class page_classes leaves out).  A row sums to 1
 * up to rounding, and the tokens of a page sum to its tq_decode_attention_mass
 * entry.  Same workspace and errors as tq_decode_attention, plus
 * TQ_ERR_INVALID_ARG for a null token_mass and TQ_ERR_ALIGNMENT for one not
 * 16-byte aligned. */
int tq_decode_attention_token_mass(const tq_layer* layer, const tq_cache* cache,
                                   const tq_query* query, float* out, float* token_mass,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* tq_decode_attention without a caller's workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The query-prep rows and split partials
 * live in a file-scope device array of the library, TQ_NOALLOC_SCRATCH_BYTES
 * bytes per GPU, allocated with the library's code object and held until the
 * process ends; its device address is looked up once per device on the first
 * call there.  The call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine) and needs nothing cleared.  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race and give wrong results; serialise them.  Returns
 * TQ_ERR_WORKSPACE when tq_decode_workspace_bytes(cache, n_q_heads) exceeds
 * TQ_NOALLOC_SCRATCH_BYTES (then nothing is launched); otherwise as
 * tq_decode_attention, with the same results bit for bit. */
#define TQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int tq_decode_attention_noalloc(const tq_layer* layer, const tq_cache* cache,
                                const tq_query* query, float* out, void* stream);

/* Dense reconstruction of tokens [tok0, tok0 + ntok) of every (session,
 * KV head): out[b][h][t][0..127] float32 (device, contiguous).  which = 0 keys,
 * 1 values; add_qjl adds the QJL residual on keys of QJL pages.  fp16 pages
 * give their stored values.  For checking the codec; not on the decode path. */
int tq_dequantize(const tq_layer* layer, const tq_cache* cache, int which,
                  int add_qjl, int tok0, int ntok, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
