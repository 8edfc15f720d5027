/*
 * tpla.h - C ABI of libtpla.so: TPLA decode attention on AMD Instinct MI355X
 * (gfx950).
 *
 * The method (arXiv 2508.15881, "TPLA: Tensor Parallel Latent Attention for
 * Efficient Disaggregated Prefill & Decode Inference"; English abstract on
 * the chatpaper.ai / fugumt.com / searcharxiv.org pages, revised abstract on
 * the paperbot-e5f.pages.dev page, and the blogs.edgentiq.com article):
 * MLA caches one low-rank latent vector cKV per token.  TPLA splits that
 * latent, and every head's input dimension (the absorbed query), across
 * tensor-parallel devices.  Each device attends over the whole sequence with
 * all heads, using only its latent slice, and the devices sum their results
 * with an all-reduce.  An orthogonal transform (Hadamard) applied to query
 * and latent before the split reduces the error between shards.  Decode is
 * memory bound, so the latent cache each device streams is the cost.
 *
 * One call of tpla_decode_shard is one device's share of one decode step:
 * every head, every sequence, one latent slice (with the whole 512-wide
 * latent it is plain MLA under tensor parallelism, the scheme TPLA is
 * compared against).  tpla_mla_prefill is the other phase: TPLA keeps the
 * MLA form for the compute-bound prefill and slices only for decode.
 *
 * Conventions for every entry point:
 *  - The caller owns all memory.  Pointers marked "device" point to GPU
 *    memory of the current HIP device.  The library allocates nothing; the
 *    decode call takes a caller-provided workspace (size query below).
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *    Every call only enqueues work on it and returns; none synchronises.
 *  - Sizes and strides are counted in elements, not bytes.
 *  - Host-visible arguments are checked before anything is enqueued; a
 *    failed check returns a non-zero status, enqueues nothing, and leaves
 *    a message for tpla_last_error().  A HIP launch error returns
 *    TPLA_ERR_HIP.  Device-resident data (block ids, positions, lengths)
 *    are not read by the host; kernels skip rows whose position or block id
 *    is out of range, so bad device data gives unspecified results but no
 *    access outside the buffers described here.
 *  - bf16 means IEEE binary32 truncated to its top 16 bits (uint16 storage);
 *    every float32 -> bf16 conversion rounds to nearest, ties to even.
 *  - No function throws; all are thread-safe (the error text is per thread).
 *
 * Choices a caller of the bare method (rotate, append, decode, combine)
 * should know about:
 *  - Argument order: every buffer is followed by its own dtype and row
 *    stride, e.g. tpla_hadamard_latent(x, x_dtype, x_row_stride, y,
 *    y_dtype, y_row_stride, rows, n, stream); n may be up to 4096.
 *    tpla_append_kv also takes `batch`, the rows of the block table, so a
 *    row naming another sequence is skipped instead of reading past the
 *    table.
 *  - Alignment: the bf16 matrix-core decode kernels need 16-byte aligned
 *    operands; a shape they serve fails with TPLA_ERR_ALIGN when the
 *    operands miss it, rather than running the float32 kernel some 400x
 *    slower.  Shapes no matrix-core kernel serves run the float32 kernel at
 *    any alignment.
 *  - Device data: there is no separate checking build.  Every kernel clamps
 *    what it reads from device memory (an out-of-range block id reads the
 *    cache's first rows, a length past max_seq_len is cut to it, a row past
 *    its sequence's blocks is skipped), at no cost to the fast path: bad
 *    data gives unspecified output and no access outside the buffers.
 *  - Enumerations are 32-bit integers; any value may be passed (checked).
 *  - Beyond the four calls: tpla_rotate_append (rotation and append in one
 *    launch), tpla_decode_suggest_splits(_cus) (split count from host-side
 *    lengths), tpla_decode_shard_noalloc (no workspace), tpla_up_project,
 *    tpla_mla_prefill.
 */
#ifndef TPLA_H_
#define TPLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums of this interface are 32-bit integers.  A caller may pass any
 * value (the library checks it): C++ sees them with int32_t as the fixed
 * underlying type, which makes every int32_t value a valid one, and C
 * compilers lay them out as int. */
#ifdef __cplusplus
#define TPLA_ENUM(name) enum name : int32_t
#else
#define TPLA_ENUM(name) enum name
#endif

typedef TPLA_ENUM(tpla_status) {
  TPLA_OK = 0,
  TPLA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  TPLA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent          */
  TPLA_ERR_ALIGN = 3,       /* pointer/stride alignment the kernel needs       */
  TPLA_ERR_DTYPE = 4,       /* unsupported element type or combination         */
  TPLA_ERR_UNSUPPORTED = 5, /* valid request no kernel of the library serves   */
  TPLA_ERR_WORKSPACE = 6,   /* workspace missing or too small                  */
  TPLA_ERR_HIP = 7          /* the HIP runtime reported an error               */
} tpla_status;

typedef TPLA_ENUM(tpla_dtype) {
  TPLA_FP32 = 0,
  TPLA_BF16 = 1
} tpla_dtype;

/*
 * tpla_hadamard_latent: y[r, :] = x[r, :] . H_n / sqrt(n) for r < rows.
 *
 * The orthogonal transform TPLA applies to the absorbed query and to the
 * latent before slicing them across devices (abstract: Hadamard before TP
 * slicing; edgentiq blog, section "How TPLA Works: Smart Slicing and
 * Reparameterization").  H_n is Sylvester's Hadamard matrix in natural
 * order (H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]), so the map is
 * orthonormal, symmetric and its own inverse: calling it on the combined
 * output rotates that back.
 *
 *  x, y        device, rows x n elements, row r at x + r*x_row_stride.
 *              x == y (same rows, same strides) is allowed; other overlaps
 *              are not.
 *  x_dtype,
 *  y_dtype     TPLA_FP32 or TPLA_BF16, any combination.  Arithmetic is
 *              float32; the result is rounded once to y_dtype.
 *  n           power of two, 1 <= n <= 4096.
 *  strides     >= n.
 * Errors: TPLA_ERR_NULL (x or y NULL with rows > 0), TPLA_ERR_SHAPE (n not
 * a power of two or > 4096, rows < 0, stride < n), TPLA_ERR_DTYPE.
 * rows == 0 is a no-op.
 */
tpla_status tpla_hadamard_latent(const void* x, tpla_dtype x_dtype, int64_t x_row_stride,
                                 void* y, tpla_dtype y_dtype, int64_t y_row_stride,
                                 int64_t rows, int32_t n, void* stream);

/*
 * tpla_append_kv: write new rows into one shard's paged latent cache.
 *
 * MLA caches only the latent cKV (plus the shared rope key); under TPLA a
 * device caches only its latent slice (abstract; paperbot revised abstract).
 * For each row t < n_rows, with b = row_seq[t] and p = row_pos[t]:
 *     slot = block_table[b*max_blocks_per_seq + p/block_size]*block_size
 *            + p % block_size
 *     cache[slot, 0:d_s]       = latent[t*latent_row_stride + 0 .. d_s)
 *     cache[slot, d_s:d_s+d_r] = rope  [t*rope_row_stride   + 0 .. d_r)
 * The caller passes `latent` already offset to its shard's columns
 * (g*d_s for shard g of a row of width d_c).
 *
 *  cache        device, [num_blocks, block_size, d_s + d_r], cache_dtype.
 *  block_table  device int32 [batch, max_blocks_per_seq].
 *  row_seq,
 *  row_pos      device int32 [n_rows].
 *  latent,rope  device, src_dtype.  rope may be NULL only if d_r == 0.
 *  Conversion: same type -> bit copy; float32 -> bf16 rounds to nearest
 *  even; bf16 -> float32 is exact.
 *  Rows with b outside [0, batch), p outside [0, max_blocks_per_seq *
 *  block_size) or a block id outside [0, num_blocks) are skipped.  Two rows
 *  that map to the same slot race.
 * Errors: TPLA_ERR_NULL, TPLA_ERR_SHAPE (non-positive sizes, n_rows < 0,
 * strides shorter than a row), TPLA_ERR_DTYPE.  n_rows == 0 is a no-op.
 */
tpla_status tpla_append_kv(void* cache, tpla_dtype cache_dtype, int32_t num_blocks,
                           int32_t block_size, int32_t d_s, int32_t d_r,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           int32_t batch, const int32_t* row_seq, const int32_t* row_pos,
                           int32_t n_rows, const void* latent, int64_t latent_row_stride,
                           const void* rope, int64_t rope_row_stride, tpla_dtype src_dtype,
                           void* stream);

/*
 * Arguments of tpla_rotate_append.
 */
typedef struct tpla_rotate_append_args {
  int32_t n;                   /* latent width d_c: power of two, 64 .. 4096    */
  const void* q;               /* device, q_rows absorbed-query rows of n       */
  tpla_dtype q_dtype;
  int64_t q_row_stride;        /* elements                                      */
  void* q_out;                 /* device, rotated query rows (may equal q)      */
  tpla_dtype q_out_dtype;
  int64_t q_out_row_stride;
  int64_t q_rows;              /* 0: no query rows                              */
  const void* latent;          /* device, n_rows new-token latent rows of n,    */
                               /*   unrotated                                   */
  const void* rope;            /* device, n_rows rope rows of d_r (NULL if 0)   */
  tpla_dtype src_dtype;        /* of latent, rope and latent_out                */
  int64_t latent_row_stride;
  int64_t rope_row_stride;
  void* latent_out;            /* device or NULL: the rotated latent rows       */
  int64_t latent_out_row_stride;
  int32_t n_rows;              /* 0: no new rows                                */
  const int32_t* row_seq;      /* device int32 [n_rows]                         */
  const int32_t* row_pos;      /* device int32 [n_rows]                         */
  void* const* caches;         /* HOST array of n_caches device shard caches    */
  int32_t n_caches;            /* 0 .. 16                                       */
  int32_t first_shard;         /* caches[c] holds latent shard first_shard + c  */
  tpla_dtype cache_dtype;
  int32_t num_blocks;          /* per cache, as tpla_append_kv                  */
  int32_t block_size;
  int32_t d_s;
  int32_t d_r;
  const int32_t* block_table;  /* device int32 [batch, max_blocks_per_seq]      */
  int32_t max_blocks_per_seq;
  int32_t batch;
  int32_t latent_norm;         /* TPLA_NORM_*: RMS norm of the rotated latent   */
  float norm_eps;              /* > 0 when latent_norm != TPLA_NORM_NONE        */
} tpla_rotate_append_args;

/* RMS normalisation of the rotated new-token latent (tpla_rotate_append). */
enum {
  TPLA_NORM_NONE = 0,          /* the latent arrives normalised                 */
  TPLA_NORM_GLOBAL = 1,        /* by the RMS of the whole rotated row           */
  TPLA_NORM_SLICE = 2          /* each d_s slice by its own RMS (RMSNorm        */
                               /*   slicing: one device's local statistics)     */
};

/*
 * tpla_rotate_append: the rotation of the query, the rotation of the new
 * token's latent and its paged append (tpla_hadamard_latent twice and
 * tpla_append_kv once per cache) in one launch, with identical results.
 *
 * TPLA rotates the absorbed query and the latent by an orthogonal transform
 * before slicing them (TPLA abstract; edgentiq blog, "How TPLA Works: Smart
 * Slicing and Reparameterization"), and each device caches only its latent
 * slice plus the rope (TPLA abstract).  With Hn = H_n / sqrt(n):
 *     q_out[r, :]      = q[r, :] . Hn                      r < q_rows
 *     c~               = N(latent[t, :] . Hn)              t < n_rows
 *     latent_out[t, :] = c~                                (if latent_out)
 *     caches[c][slot]  = [ c~[(first_shard+c)*d_s : +d_s] || rope[t, :] ]
 * with slot as in tpla_append_kv (rows with an out-of-range sequence,
 * position or block id are skipped).  N is the identity (TPLA_NORM_NONE),
 * y / sqrt(mean(y^2) + norm_eps) over the whole row (TPLA_NORM_GLOBAL), or
 * the same over each block of d_s columns on its own (TPLA_NORM_SLICE):
 * the RMSNorm slicing of the edgentiq blog's "How TPLA Works" section, in
 * which a device normalises its latent slice with that slice's own
 * statistics and the rotation before the split keeps them close to the
 * global ones.  The norm's gain is left to the weights that read the
 * latent.  Arithmetic and rounding are those of tpla_hadamard_latent
 * (float32, one round-to-nearest-even to the output dtype, after the
 * norm); a rope of the cache's type is copied bit for bit.  The query rows
 * are never normalised.
 * Errors: TPLA_ERR_NULL, TPLA_ERR_SHAPE (n not a power of two in
 * [64, 4096], strides shorter than a row, shards beyond n, n_caches outside
 * [0, 16], negative counts, latent_norm unknown, norm_eps not a positive
 * finite number when a norm is asked for, TPLA_NORM_SLICE with d_s outside
 * [1, n]), TPLA_ERR_UNSUPPORTED (TPLA_NORM_SLICE with d_s not a power of
 * two or below n / 64), TPLA_ERR_DTYPE.
 */
tpla_status tpla_rotate_append(const tpla_rotate_append_args* args, void* stream);

/*
 * Arguments of one shard's decode step (see tpla_decode_shard).
 */
typedef struct tpla_decode_args {
  int32_t batch;               /* sequences                                     */
  int32_t heads;               /* query heads; all of them run on every shard   */
  int32_t d_s;                 /* latent slice width of this shard (d_c / tp)   */
  int32_t d_r;                 /* rope width (0 allowed)                        */
  int32_t block_size;          /* cache rows per physical block                 */
  int32_t num_blocks;          /* physical blocks in `cache`                    */
  int32_t max_blocks_per_seq;  /* columns of `block_table`                      */
  int32_t max_seq_len;         /* host-side bound: seq_lens[b] <= max_seq_len   */
  tpla_dtype dtype;            /* element type of q_latent, q_rope and cache    */
  float scale;                 /* softmax scale applied to the whole score      */
  const void* q_latent;        /* device, absorbed query slice; element (b,h,k) */
  int64_t q_latent_stride_b;   /*   at q_latent + b*stride_b + h*stride_h + k   */
  int64_t q_latent_stride_h;
  const void* q_rope;          /* device, rope query, (b,h,k) as above          */
  int64_t q_rope_stride_b;
  int64_t q_rope_stride_h;
  const void* cache;           /* device, [num_blocks, block_size, d_s + d_r]   */
  const int32_t* block_table;  /* device int32 [batch, max_blocks_per_seq]      */
  const int32_t* seq_lens;     /* device int32 [batch], tokens to attend over   */
  void* out;                   /* device, (b,h,k) at out + b*sb + h*sh + k      */
  tpla_dtype out_dtype;
  int64_t out_stride_b;
  int64_t out_stride_h;
  float* lse;                  /* device float32 [batch, heads] or NULL         */
  int32_t num_splits;          /* token splits per sequence; 0 = automatic.     */
                               /* A request: raised where a kernel caps the     */
                               /* tokens of one split (65536 on the bf16        */
                               /* streaming kernels).  Automatic on the 128-    */
                               /* head d_s = 256 kernel: units of equal tiles   */
                               /* cut from the lengths on the device (see       */
                               /* tpla_decode_shard)                            */
} tpla_decode_args;

/*
 * tpla_decode_workspace_size: bytes of device workspace tpla_decode_shard
 * needs for `args` (same args => same size, on the same device).
 * Errors: as tpla_decode_shard's argument checks; TPLA_ERR_HIP if the device
 * cannot be queried.
 */
tpla_status tpla_decode_workspace_size(const tpla_decode_args* args, size_t* bytes);

/*
 * tpla_decode_suggest_splits: a value for args->num_splits chosen from the
 * host's copy of the sequence lengths (seq_lens_host[b], b < batch: the
 * same lengths the device array holds).  The automatic split count sees
 * only max_seq_len, which for a ragged batch leaves many splits empty and a
 * few long ones; this one models a launch of the streaming kernel (work
 * units in launch order, their XCD, one workgroup per CU, a fixed
 * start and finish per unit) and returns the count with the shortest
 * modelled launch, preferring fewer splits on ties.  For shapes that do not
 * run the streaming kernel it returns the automatic count, and for the
 * 128-head d_s = 256 and 64-head d_s = 128 kernels, whose automatic plan
 * balances units over the device's lengths itself, it returns 0
 * (automatic).  It reads
 * nothing on the device and launches nothing; args->num_splits is ignored.
 * Errors: as tpla_decode_workspace_size; TPLA_ERR_NULL for a NULL
 * seq_lens_host or num_splits.
 */
tpla_status tpla_decode_suggest_splits(const tpla_decode_args* args, const int32_t* seq_lens_host,
                                       int32_t* num_splits);

/*
 * tpla_decode_suggest_splits_cus: the same suggestion for a device with
 * `cus` compute units, without querying any device (a scheduler planning
 * for a GPU it does not drive; tests on a host without one).
 * Errors: as tpla_decode_suggest_splits; TPLA_ERR_SHAPE for cus < 1.
 */
tpla_status tpla_decode_suggest_splits_cus(const tpla_decode_args* args,
                                           const int32_t* seq_lens_host, int32_t cus,
                                           int32_t* num_splits);

/*
 * tpla_decode_shard: one device's share of a TPLA decode step.
 *
 * Per-shard attention with the shard's own softmax (abstract: attention is
 * performed independently per shard; edgentiq blog, "How TPLA Works": the
 * global score is approximated from local computations).  For every
 * sequence b < batch and head h < heads, with L = seq_lens[b] and the
 * cache row of logical token j read through the block table,
 *     s_j  = scale * ( q_latent[b,h,:] . row_j[0:d_s]
 *                    + q_rope[b,h,:]   . row_j[d_s:d_s+d_r] )
 *     out[b,h,:] = sum_j softmax(s)_j * row_j[0:d_s]
 *     lse[b,h]   = log sum_j exp(s_j)
 * The rope part is whole on every shard; only the latent is sliced.
 * L == 0 gives out = 0 and lse = -inf.  Tokens j >= L are never read.
 *
 * The work is split over tokens; each split keeps a running max and sum
 * (online softmax) and the splits are merged by log-sum-exp before `out` is
 * written.  On the d_s = 256 (heads % 128 == 0) and d_s = 128 (heads % 64
 * == 0) kernel the splits are work units derived on the device from
 * seq_lens: with num_splits = 0, sequence b's ceil(L_b / 64) tiles are cut
 * into units of c tiles, c the smallest chunk that leaves at most one unit
 * per CU and head group (capped at 1024 tiles), so a ragged
 * batch gives every CU about the same work; with num_splits > 0 the chunk
 * is the uniform one of that many splits of max_seq_len.
 *
 * Kernels: with dtype BF16, 16-byte aligned q_latent/q_rope/cache and query
 * strides that are multiples of 8,
 *   - the streaming matrix-core kernel serves block_size % 64 == 0, d_r == 64
 *     and either heads % 128 == 0 with d_s == 256 or heads % 64 == 0 with
 *     d_s == 128;
 *   - a streaming matrix-core kernel for the whole 512-wide latent serves
 *     d_s == 512, d_r == 64, heads % 16 == 0 and block_size % 32 == 0: plain
 *     MLA under tensor parallelism (every device keeps the whole latent for
 *     its heads; TPLA abstract), or one shard at T = 1;
 *   - a register-staged matrix-core kernel serves heads % 32 == 0 with d_s
 *     in {64, 128, 256} and d_r in {0, 64};
 * a bf16 shape that one of these serves but whose operands miss the
 * alignment above fails with TPLA_ERR_ALIGN (the float32 kernel would take
 * it some 400x slower); every other case (and FP32) runs a float32 kernel,
 * which needs
 * 4*(24*(d_s + d_r) + 8*d_s + 152) <= 65536 bytes of LDS (e.g. d_s = 256,
 * d_r = 64 fits; d_s = 512, d_r = 64 does not: TPLA_ERR_UNSUPPORTED there).
 * out_dtype FP32 or BF16.
 * workspace: device, at least tpla_decode_workspace_size() bytes, 256-byte
 * aligned; its contents on entry do not matter.  The split outputs go there
 * (fp16 with a float scale per 64 columns on the streaming kernels, float32
 * otherwise) and a second kernel on the same stream merges them into `out`.
 * Errors: TPLA_ERR_NULL, TPLA_ERR_SHAPE, TPLA_ERR_ALIGN (bf16 operands or
 * workspace misaligned, above), TPLA_ERR_DTYPE, TPLA_ERR_UNSUPPORTED (no
 * kernel for the shape, above), TPLA_ERR_WORKSPACE, TPLA_ERR_HIP.
 */
tpla_status tpla_decode_shard(const tpla_decode_args* args, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * tpla_decode_shard_noalloc: tpla_decode_shard without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split outputs go to a static device array of the library,
 * tpla_decode_noalloc_scratch_bytes() bytes (64 MiB) on every device it
 * runs on, held until the process ends; the call allocates nothing.  The
 * first call on a device looks up that device's copy
 * (hipGetSymbolAddress) with the device current, so make the stream's
 * device the current one.  Same kernels, same results as tpla_decode_shard
 * with a workspace.  Nothing in the scratch needs to start at zero.
 * Calls that overlap on one device (other streams, other threads) share the
 * one array and race: order them on one stream or serialise them.
 * Errors: as tpla_decode_shard; TPLA_ERR_WORKSPACE when the call's split
 * outputs (tpla_decode_workspace_size) exceed the scratch;
 * TPLA_ERR_UNSUPPORTED for a device index of 64 or more.
 */
tpla_status tpla_decode_shard_noalloc(const tpla_decode_args* args, void* stream);

/* tpla_decode_noalloc_scratch_bytes: size of that static scratch, bytes. */
size_t tpla_decode_noalloc_scratch_bytes(void);


/*
 * tpla_up_project: one device's value up-projection, optionally added into
 * an output that already holds other devices' terms:
 *     y[b, h, v] = (accumulate ? y[b, h, v] : 0) + sum_k o[b, h, k] * w[h, v, k]
 * for b < batch, h < heads, v < d_v, k < d_s.
 *
 * Under TPLA a device's attention output o covers only its latent slice;
 * the head's output is the sum over devices of W_UV's matching columns
 * times o, and that sum is the all-reduce (TPLA abstract: per-shard
 * attention combined with an all-reduce; paperbot revised abstract: the
 * orthogonal reparameterisation keeps MLA's weights usable).  w is W_UV in
 * its own layout ([head][v][latent]) restricted to the device's latent
 * columns (w_stride_v = the full latent width for a column slice); with a
 * rotated latent (tpla_hadamard_latent) it is W_UV . Hn.  On one device the
 * all-reduce is the accumulation of the devices' calls into one y.
 *
 *  o   device, element (b, h, k) at o + b*o_stride_b + h*o_stride_h + k.
 *  w   device, element (h, v, k) at w + h*w_stride_h + v*w_stride_v + k.
 *  y   device, element (b, h, v) at y + b*y_stride_b + h*y_stride_h + v;
 *      must not overlap o or w.
 *  dtypes  TPLA_FP32 or TPLA_BF16 each.  The products are exact (float32
 *      operands are split into three bf16 terms on the matrix cores) and
 *      summed in float32; one rounding to y's type, after the addition of
 *      the old value when accumulating.
 * Requirements: batch, heads, d_s, d_v >= 1; heads <= 65535; batch <=
 * 2097120; o_stride_h >= d_s, w_stride_v >= d_s, w_stride_h >= d_v *
 * w_stride_v, y_stride_h >= d_v, batch strides >= 0.
 * Errors: TPLA_ERR_NULL, TPLA_ERR_SHAPE, TPLA_ERR_DTYPE, TPLA_ERR_HIP.
 */
tpla_status tpla_up_project(const void* o, tpla_dtype o_dtype, int64_t o_stride_b,
                            int64_t o_stride_h, const void* w, tpla_dtype w_dtype,
                            int64_t w_stride_h, int64_t w_stride_v, void* y, tpla_dtype y_dtype,
                            int64_t y_stride_b, int64_t y_stride_h, int32_t batch, int32_t heads,
                            int32_t d_s, int32_t d_v, int32_t accumulate, void* stream);

/*
 * tpla_combine_shards: the all-reduce of the shard outputs, on one device.
 *
 * Shards hold disjoint latent columns, so the sum of the zero-padded shard
 * outputs is their placement side by side (abstract: results are combined
 * with an all-reduce):
 *     out[b, h, g*d_s + k] = (accumulate ? out[b, h, g*d_s + k] : 0)
 *                            + partials[g][(b*heads + h)*d_s + k]
 * partials: HOST array of tp device pointers, each [batch, heads, d_s]
 * contiguous, part_dtype.  out: device [batch, heads, tp*d_s] contiguous.
 * With accumulate == 0 the values are copied (bit exact for equal types,
 * nearest-even for float32 -> bf16).
 * Errors: TPLA_ERR_NULL, TPLA_ERR_SHAPE (tp outside [1, 16], sizes < 1),
 * TPLA_ERR_DTYPE.
 */
tpla_status tpla_combine_shards(const void* const* partials, tpla_dtype part_dtype, int32_t tp,
                                int32_t batch, int32_t heads, int32_t d_s, void* out,
                                tpla_dtype out_dtype, int32_t accumulate, void* stream);

/*
 * Arguments of an MLA-form prefill (see tpla_mla_prefill).
 */
typedef struct tpla_prefill_args {
  int32_t batch;               /* prompts                                       */
  int32_t heads;               /* query heads on this device                    */
  int32_t d_c;                 /* latent width: 512                             */
  int32_t d_r;                 /* rope width: 64                                */
  int32_t max_len;             /* positions per prompt in the buffers below     */
  tpla_dtype dtype;            /* element type of q_latent, q_rope, kv: BF16    */
  float scale;                 /* softmax scale applied to the whole score      */
  const void* q_latent;        /* device, absorbed query; element (b,t,h,k) at  */
  int64_t q_latent_stride_b;   /*   q_latent + b*stride_b + t*stride_t          */
  int64_t q_latent_stride_t;   /*   + h*stride_h + k                            */
  int64_t q_latent_stride_h;
  const void* q_rope;          /* device, rope query, (b,t,h,k) as above        */
  int64_t q_rope_stride_b;
  int64_t q_rope_stride_t;
  int64_t q_rope_stride_h;
  const void* kv;              /* device, prompt rows [latent (d_c) || rope key */
  int64_t kv_stride_b;         /*   (d_r)]: row (b,t) at kv + b*stride_b +      */
  int64_t kv_stride_t;         /*   t*stride_t, d_c + d_r contiguous elements   */
  const int32_t* seq_lens;     /* device int32 [batch], prompt lengths          */
  void* out;                   /* device, (b,t,h,k) at out + b*sb + t*st + h*sh */
  tpla_dtype out_dtype;        /*   + k; FP32 or BF16                           */
  int64_t out_stride_b;
  int64_t out_stride_t;
  int64_t out_stride_h;
  float* lse;                  /* device float32 [batch, max_len, heads] or NULL */
} tpla_prefill_args;

/*
 * tpla_mla_prefill: attention of every prompt position over the prompt, in
 * the MLA form (no slicing, no rotation).  TPLA keeps MLA for the
 * compute-bound prefill and switches to the sliced form for decode
 * (paperbot revised abstract; edgentiq blog, "Prefill-Decode Separation for
 * Optimal Performance"); the prompt's rows reach the shard caches through
 * tpla_rotate_append, like decode's new rows.
 *
 * For b < batch, t < seq_lens[b] and every head h (causal: positions 0..t):
 *     s_j = scale * (q_latent[b,t,h,:] . kv[b,j,0:d_c]
 *                    + q_rope[b,t,h,:] . kv[b,j,d_c:d_c+d_r]),  j <= t
 *     out[b,t,h,:] = sum_j softmax(s)_j * kv[b,j,0:d_c]
 *     lse[b,t,h]   = log sum_j exp(s_j)                 (if lse != NULL)
 * Positions t >= seq_lens[b] (clamped to [0, max_len]) are not written.
 *
 * Layout: q_latent, q_rope and kv 16-byte aligned with strides that are
 * multiples of 8 elements; out 16-byte aligned with strides that are
 * multiples of 4 elements; kv_stride_t >= d_c + d_r and below 2^26.
 * Kernel: bf16 matrix cores.  With heads a multiple of 64, one workgroup of
 * eight waves per (prompt, position, 64 heads), score and value waves
 * apart; otherwise one workgroup of four waves per 64 (position, head) rows.
 * Errors: TPLA_ERR_NULL, TPLA_ERR_SHAPE, TPLA_ERR_ALIGN, TPLA_ERR_DTYPE,
 * TPLA_ERR_UNSUPPORTED (d_c != 512 or d_r != 64), TPLA_ERR_HIP.
 */
tpla_status tpla_mla_prefill(const tpla_prefill_args* args, void* stream);

/* Static text for a status code: a tpla_status value, passed as an
 * integer so that any value is valid ("unknown status" outside the enum). */
const char* tpla_status_string(int32_t status);
/* Message of the last failed call on this thread ("" if none). */
const char* tpla_last_error(void);
/* Library version as major*10000 + minor*100 + patch. */
int32_t tpla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TPLA_H_ */
