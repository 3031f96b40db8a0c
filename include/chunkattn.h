/*
 * chunkattn -- chunked spatio-temporal attention for a DualParal-style FIFO
 * chunk queue on AMD Instinct MI355X (gfx950).  C ABI: plain pointers and
 * sizes, no C++ types, no exceptions across the boundary.
 *
 * The operation (cited by page and section):
 *
 *   DualParal write-up, techwalker.com, "双重并行：让AI视频生成突破时长限制",
 *   section 二 (FIFO queue and block-wise denoising): the video is cut into
 *   fixed-size, non-overlapping temporal chunks held in a FIFO queue, every
 *   chunk at its own noise level, all of them processed in one step and fed
 *   from the tail to the head.  Section 三 (feature cache): the self-attention
 *   K/V of the chunk processed just before are kept and reused by the next
 *   chunk, so no concatenated copy of the neighbouring chunk is built; only
 *   self-attention uses the cache, cross-attention stays per chunk.
 *   Video-diffusion survey, intelliparadigm.com, "视频扩散模型：核心技术挑战与
 *   前沿进展", section 2.1 item 2: spatio-temporal attention attends jointly
 *   over all tokens of the frames in its window.
 *
 * Reading.  Chunk c (0-based, processing order) attends over
 *   R_c = [predecessor K/V: chunk c-1's rows 0..L-1, only if c >= 1] ++ [own rows 0..L-1]
 * with plain softmax attention, no mask inside R_c:
 *   O[c,r,h,:] = softmax_j(scale * <Q[c,r,h,:], K_j[h,:]>) . V_j[h,:]
 * Chunk 0 has a zero-length cache.
 *
 * Layouts (row-major, element = one bf16 or fp32 value):
 *   q, k, v, out : [n_chunks][chunk_len][heads][head_dim]   (token-major, as a
 *                  DiT's activations; a chunk's tokens are frame-major f,y,x,
 *                  which attention does not depend on)
 *   kv_cache     : [n_chunks][2][chunk_len][heads][head_dim]; slot c holds the
 *                  predecessor's K (index 0) then V (index 1); slot 0 is never read.
 *
 * Numerics.  bf16 calls: Q.K^T and P.V run on bf16 matrix cores with fp32
 * accumulation and an fp32 softmax; P is rounded to bf16 before the P.V
 * product and the softmax denominator is summed from the same rounded P, so a
 * constant V comes back bit-exactly.  With 256- and 384-row work items Q is
 * multiplied by scale * log2 e and rounded to bf16 once per item (relative
 * 2^-9 per element).  bf16 outputs are rounded nearest-even.  fp32 calls
 * (dtype F32) keep fp32 throughout: fp32 matrix cores, an fp32 softmax with a
 * running maximum, fp32 output (64-row work items; the fp32 matrix-core peak
 * is a sixteenth of the bf16 one).  Results are bitwise deterministic run to run, and the
 * separate-cache and in-place-predecessor forms give bitwise-equal outputs.
 *
 * Ownership and asynchrony.  Every tensor pointer is device memory owned by the
 * caller and must stay valid until the stream work completes.  The library
 * owns only the context; a context also owns a 64 KB device buffer, 512
 * work-queue slots of its persistent main passes (256- and 384-row items),
 * allocated by chunkattn_create, and a stream-ordered memory pool from which a
 * launch with few items per CU takes the workspace of its key-axis split (see
 * chunkattn_ctx_set_tail_split; the pool keeps its memory, so a call
 * allocates only while the pool grows).  The calls validate, enqueue the
 * kernels on hip_stream (NULL = the legacy default stream) and return; a
 * device fault surfaces at the caller's next synchronisation.  One context may
 * be used by one host thread at a time; separate contexts are independent.
 * Each call with a persistent main pass uses one work-queue slot, which a
 * small kernel on hip_stream clears right before the main pass.  Eager calls take the next of 64 slots in turn: calls may be
 * spread over several streams as long as at most 64 of them are in flight at
 * once (calls on one stream never overlap).  A call made while hip_stream is
 * being captured into a graph gets a slot of its own (at most 448 such calls
 * per context; the next one fails with CHUNKATTN_EUNSUPPORTED), which only
 * that graph's replays use: replays of different graphs may overlap each
 * other and eager calls; replays of one graph must not overlap each other
 * (launches of one executable graph are ordered).
 *
 * Sizes.  heads * head_dim * element size * 64 must stay below 2^32 (the
 * kernels address a 64-row key/value tile by 32-bit byte offsets); larger
 * rows fail with CHUNKATTN_EUNSUPPORTED.
 *
 * Errors.  Every call returns a chunkattn_status synchronously, before any
 * launch, for bad arguments; chunkattn_last_error() then holds a one-line
 * explanation.  Nothing in the library calls exit() or abort().
 */
#ifndef CHUNKATTN_H
#define CHUNKATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct chunkattn_ctx chunkattn_ctx; /* opaque, library-owned */

typedef enum {
    CHUNKATTN_OK = 0,
    CHUNKATTN_EINVAL = 1,       /* bad argument: null/misaligned pointer, size, aliasing */
    CHUNKATTN_EUNSUPPORTED = 2, /* head_dim, dtype or device not supported */
    CHUNKATTN_EDEVICE = 3,      /* HIP runtime error outside a launch */
    CHUNKATTN_ENOMEM = 4,       /* host allocation of the context failed */
    CHUNKATTN_ELAUNCH = 5       /* the kernel launch was rejected */
} chunkattn_status;

typedef enum {
    CHUNKATTN_BF16 = 0, /* bf16 storage in and out */
    CHUNKATTN_F32 = 1   /* fp32 storage in and out, fp32 arithmetic */
} chunkattn_dtype;

/* chunkattn_create flags: query rows per work item (one workgroup) of bf16
 * calls.  With no flag (0) a context uses 384-row items for head_dim-128 calls
 * and 256-row items for head_dim 64; CHUNKATTN_FLAG_BLOCK384 asks for the same
 * explicitly.  fp32 calls always use 64-row items on the fp32 kernel. */
#define CHUNKATTN_FLAG_BLOCK128 1u /* 128 rows, 4 waves, two workgroups per CU */
#define CHUNKATTN_FLAG_BLOCK256 2u /* 256 rows, 8 waves of 32 rows, one workgroup per CU */
#define CHUNKATTN_FLAG_BLOCK384 4u /* 384 rows, 8 waves of 48 rows, one workgroup per CU,
                                      for bf16 head_dim 128 (256 rows otherwise) */
/* Exact scale (may be or-ed with CHUNKATTN_FLAG_BLOCK384 or BLOCK128).  The
 * default 384- and 256-row passes round scale * log2(e) * Q to bf16 once per
 * work item, which adds a relative error of up to 2^-9 to every score term:
 * harmless for near-uniform softmax rows, but it grows with the spread of the
 * logits (natural-logit standard deviation 5 gives max-abs output errors near
 * 2e-2 against 1e-2 for exact scaling).  With this flag the scores are scaled
 * in fp32 instead: 384-row items multiply S by scale * log2(e) (about 6% more
 * time), calls without the 384-row kernel use 128-row items (which always
 * scale in fp32).  CHUNKATTN_EINVAL together with CHUNKATTN_FLAG_BLOCK256. */
#define CHUNKATTN_FLAG_EXACT_SCALE 8u

/* Query rows per work item of a bf16, head_dim-128 call on a context created
 * with flags = 0 (384). */
int chunkattn_block_rows(void);

/*
 * Creates a context bound to HIP device `device_ordinal`.  Fails with
 * CHUNKATTN_EUNSUPPORTED unless the device is gfx950, CHUNKATTN_EDEVICE if the
 * ordinal is invalid.  `flags` is 0 (library default work-item size) or one of
 * CHUNKATTN_FLAG_BLOCK128 / CHUNKATTN_FLAG_BLOCK256 / CHUNKATTN_FLAG_BLOCK384,
 * optionally or-ed with CHUNKATTN_FLAG_EXACT_SCALE; results do not depend on
 * the work-item size beyond fp32 rounding order.  On success *out owns the context; release it
 * with chunkattn_destroy.  CHUNKATTN_EDEVICE also reports a failed allocation
 * of the work queue (every context but a 128-row one: the 256- and 384-row
 * main passes are persistent).
 */
int chunkattn_create(chunkattn_ctx **out, int device_ordinal, unsigned flags);

/* Query rows per work item of this context for a bf16, head_dim-128 call
 * (128, 256 or 384). */
int chunkattn_ctx_block_rows(const chunkattn_ctx *ctx);

/* Query rows per work item of this context for a call with the given
 * head_dim and dtype (64 for every fp32 call). */
int chunkattn_ctx_call_block_rows(const chunkattn_ctx *ctx, int head_dim, int dtype);

/* 384-row query blocks per work item of the context's calls that use 384-row
 * blocks (bf16, head_dim 128).  A work item of several blocks of one (chunk,
 * head) walks the chunk's key/value tiles once per block as one continuous
 * stream, which spares short key walks (cross-attention over text tokens) the
 * per-item start and finish.  blocks = 0 (the default) chooses per call:
 * about 48 key tiles per item while the launch keeps at least 4 items per CU;
 * 1..8 fixes the count.  Results are the same up to fp32 rounding order for
 * every setting.  CHUNKATTN_EINVAL outside [0, 8].  Not thread-safe against
 * concurrent calls on the same context. */
int chunkattn_ctx_set_item_blocks(chunkattn_ctx *ctx, int blocks);

/* Key-axis split of the last work items of the context's calls with one
 * 384-row block per item.  A launch with few items per CU ends when its last
 * items do; cutting `items` items into `parts` ranges of their key tiles lets
 * the CUs finish together.  The items cut are the last of those with a
 * predecessor segment (the long ones; the short items of the queue's first
 * chunk stay whole and run before the parts), or the last of the launch when
 * no item has a predecessor.  Each part stores its
 * unnormalised O and row sums l (the softmax has no maximum, so the parts add
 * exactly up to fp32 rounding order) in a workspace taken from a
 * stream-ordered memory pool of the context, and the last part to finish adds
 * the others and writes the output.  items = -1 (the default): chosen per
 * call when a launch has fewer than 8 items per CU (2/3 n_CU items into 2
 * parts below 3 items per CU, n_CU items into 4 parts from 3 up); 0: never;
 * > 0: that many items, with
 * parts in [2, 8] (fewer if an item has fewer key tiles).  Never used under
 * graph capture or by chunkattn_queue_step_noalloc.  CHUNKATTN_EINVAL
 * otherwise.  Not thread-safe against concurrent calls on the same context. */
int chunkattn_ctx_set_tail_split(chunkattn_ctx *ctx, int items, int parts);

/* Releases a context (NULL is accepted). */
int chunkattn_destroy(chunkattn_ctx *ctx);

/*
 * One queue step: every chunk c in [0, n_chunks) attends over R_c (see above),
 * for every head and query row, in one launch on hip_stream.
 *
 *   q, k, v   [n_chunks][chunk_len][heads][head_dim], device, 16-byte aligned.
 *   kv_cache  [n_chunks][2][chunk_len][heads][head_dim] separate predecessor
 *             cache, or NULL to read chunk c-1's K/V from k and v in place.
 *   out       same shape and dtype as q; must not overlap any input.
 *   chunk_len, n_chunks  >= 0 (either 0: nothing to do, returns OK).
 *   heads >= 1; head_dim 64 or 128; scale finite and >= 0 (applied to Q.K^T
 *   before the softmax; 1/sqrt(head_dim) is the usual value).
 *   dtype     chunkattn_dtype of q, k, v, kv_cache and out.
 *   hip_stream  hipStream_t, or NULL.
 */
int chunkattn_queue_step(chunkattn_ctx *ctx, const void *q, const void *k, const void *v,
                         const void *kv_cache, void *out, int chunk_len, int n_chunks,
                         int heads, int head_dim, float scale, int dtype, void *hip_stream);

/*
 * For callers that cannot allocate device memory on the hot path (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same queue step as chunkattn_queue_step, same arguments, layouts, errors and
 * bit-identical results, except that the persistent main pass keeps its work
 * queue in a static device array of the library (16 words, 128 bytes per
 * device, held until the process ends) instead of the context's buffer.  The
 * call allocates nothing, host or device.  The array's device address is
 * looked up once per context by chunkattn_create.  All calls of this entry
 * point on one device share that array, which a small kernel on hip_stream
 * clears before every main pass: such calls must not overlap on one device
 * (on different streams without ordering, or graph replays running at once),
 * or they race.  Fails with CHUNKATTN_EUNSUPPORTED if the device has more
 * dies than the array has claim words (16).
 */
int chunkattn_queue_step_noalloc(chunkattn_ctx *ctx, const void *q, const void *k,
                                 const void *v, const void *kv_cache, void *out,
                                 int chunk_len, int n_chunks, int heads, int head_dim,
                                 float scale, int dtype, void *hip_stream);

/*
 * One window step, the form the feature cache is introduced for in the
 * DualParal write-up (section 三): processing the window [B_{i-1}, B_i] of
 * two neighbouring chunks reuses the cached self-attention K/V of B_{i+1},
 * the chunk processed just before.  With chunks in processing order, window c
 * (c in [0, n_chunks)) is centred on chunk c:
 *   queries  the rows of chunk c, then of chunk c+1 (2 * chunk_len rows; only
 *            chunk c's for the last window, c = n_chunks-1);
 *   keys/values  W_c = [chunk c-1's K/V from the cache (c >= 1)]
 *            ++ [own K/V of chunk c] ++ [own K/V of chunk c+1 (c+1 < n_chunks)];
 * plain softmax attention of every query row over W_c, every head, in one
 * launch on hip_stream.
 *
 *   q, k, v, kv_cache  as for chunkattn_queue_step (kv_cache slot c holds
 *            chunk c-1's K then V; NULL reads chunk c-1 in place).
 *   out      [n_chunks][2][chunk_len][heads][head_dim]: out[c][0] = window c's
 *            rows of chunk c, out[c][1] = its rows of chunk c+1.  out[n-1][1]
 *            is not written.  Must not overlap any input.
 *   chunk_len <= 2^29; other arguments as for chunkattn_queue_step.
 */
int chunkattn_window_step(chunkattn_ctx *ctx, const void *q, const void *k, const void *v,
                          const void *kv_cache, void *out, int chunk_len, int n_chunks,
                          int heads, int head_dim, float scale, int dtype, void *hip_stream);

/*
 * Streaming queue (DualParal write-up, section 二): new noisy chunks enter at
 * the tail, clean chunks leave at the head, every step processes the whole
 * queue tail first, and the video can grow without bound.  The chunks live in
 * caller-owned ring buffers of `slots` chunk slots; nothing is copied when the
 * queue advances.
 *
 * chunkattn_ring_step: one queue step over n_live chunks of a ring.  With the
 * live chunks in processing order (c = 0 the tail, the newest), chunk c is in
 * slot (tail_slot - c) mod slots; it attends over R_c = [its predecessor's
 * K/V, read in place from the slot of chunk c-1 (c >= 1)] ++ [its own K/V],
 * exactly as chunkattn_queue_step, and its output goes to the same slot of
 * out_ring.  Other slots of out_ring are not written.
 *
 *   q_ring, k_ring, v_ring, out_ring  [slots][chunk_len][heads][head_dim],
 *            device, 16-byte aligned; out_ring must not overlap an input.
 *   slots >= 1; 0 <= tail_slot < slots; 0 <= n_live <= slots (0: no-op).
 *   Other arguments as for chunkattn_queue_step.
 */
int chunkattn_ring_step(chunkattn_ctx *ctx, const void *q_ring, const void *k_ring,
                        const void *v_ring, void *out_ring, int slots, int tail_slot,
                        int n_live, int chunk_len, int heads, int head_dim, float scale,
                        int dtype, void *hip_stream);

/*
 * Host-side queue bookkeeping for chunkattn_ring_step.  Chunk number g (in
 * order of arrival, from 0) lives in slot g mod slots; a chunk spends exactly
 * `depth` steps in the queue (one per noise level), so at most depth chunks
 * are live and slots >= depth keeps them in distinct slots.  A queue object is
 * used by one host thread at a time.  Failures return a status; the
 * explanation is in chunkattn_last_error(NULL).
 */
typedef struct chunkattn_fifo chunkattn_fifo;

/* New empty queue; needs depth >= 1 and slots >= depth. */
int chunkattn_fifo_create(chunkattn_fifo **out, int slots, int depth);
int chunkattn_fifo_destroy(chunkattn_fifo *f);
/* A new chunk joins at the tail; *slot receives its slot, which the caller
 * fills with the chunk's Q/K/V.  CHUNKATTN_EINVAL if depth chunks are live. */
int chunkattn_fifo_push(chunkattn_fifo *f, int *slot);
/* The head chunk leaves; *slot receives its slot (its last output is final).
 * CHUNKATTN_EINVAL unless the head has done all depth steps. */
int chunkattn_fifo_pop(chunkattn_fifo *f, int *slot);
/* The live chunks in processing order (tail first): chunk numbers, slots and
 * steps done, at most cap of each (any of the three arrays may be NULL);
 * *n_live receives the count. */
int chunkattn_fifo_live(const chunkattn_fifo *f, long long *ids, int *slots, int *steps_done,
                        int cap, int *n_live);
/* Every live chunk has done one more step, without a launch: for callers that
 * run chunkattn_ring_step themselves (tail = slot of live chunk 0, n_live).
 * CHUNKATTN_EINVAL if the queue is empty. */
int chunkattn_fifo_advance(chunkattn_fifo *f);
/* One diffusion step of the attention over every live chunk
 * (chunkattn_ring_step with the queue's tail and count), after which every
 * live chunk has done one more step.  CHUNKATTN_EINVAL if the queue is empty;
 * on any failure the queue is unchanged. */
int chunkattn_fifo_step(chunkattn_ctx *ctx, chunkattn_fifo *f, const void *q_ring,
                        const void *k_ring, const void *v_ring, void *out_ring, int chunk_len,
                        int heads, int head_dim, float scale, int dtype, void *hip_stream);

/*
 * Coordinated noise initialization of a new chunk (DualParal write-up,
 * section 三, second improvement): the new chunk's n_frames noise frames come
 * from a shared pool of pool_frames frames, leaving out the frames used by the
 * last n_excl latent frames of the tail chunk (its temporal neighbour, NumC/2
 * in the write-up), in a random order given by the caller's keys.
 *
 *   pool      [pool_frames][frame_bytes] device memory, 16-byte aligned;
 *             frame_bytes a positive multiple of 16 (any element type: frames
 *             are copied bit for bit).  1 <= pool_frames <= 4096.
 *   keys      pool_frames uint32 on the device: the draw.  The candidates
 *             (pool frames not excluded) in ascending (key, pool index) order
 *             give the new frames: frame f is the candidate of rank f.
 *   prev_idx  the tail chunk's pool indices in frame order (n_prev ints on the
 *             device; NULL with n_prev = 0 for the first chunk); its last
 *             n_excl entries are excluded (0 <= n_excl <= n_prev; values
 *             outside [0, pool_frames) exclude nothing).
 *   out       [n_frames][frame_bytes] device, 16-byte aligned: the new noise.
 *   idx_out   n_frames ints on the device: the pool index of each new frame
 *             (the next call's prev_idx).
 *   Requires pool_frames - n_excl >= n_frames.  No output may overlap an
 *   input.  Two launches on hip_stream.
 */
int chunkattn_noise_init(chunkattn_ctx *ctx, const void *pool, int pool_frames,
                         long long frame_bytes, const void *keys, const void *prev_idx,
                         int n_prev, int n_excl, int n_frames, void *out, void *idx_out,
                         void *hip_stream);
int chunkattn_validate_noise_init(const void *pool, int pool_frames, long long frame_bytes,
                                  const void *keys, const void *prev_idx, int n_prev,
                                  int n_excl, int n_frames, const void *out,
                                  const void *idx_out);

/*
 * Non-chunked attention: every query row of batch item b attends over all lkv
 * rows of its K/V (the full-sequence attention the chunked form avoids, and
 * the per-chunk cross-attention to text tokens, which uses no cache).
 *
 *   q, out  [batch][lq][heads][head_dim]
 *   k, v    batch item b at element offset b * kv_batch_stride, each
 *           [lkv][heads][head_dim]; kv_batch_stride = 0 shares one K/V
 *           (e.g. one prompt's text tokens) across the batch.  A shared K/V
 *           runs the work items head by head (all batch items of a head
 *           together, so that each die's L2 holds few heads' K/V); the
 *           order changes no result, since every output row is computed by
 *           one work item.
 *   batch, lq >= 0 (either 0: returns OK); lkv >= 1; kv_batch_stride >= 0.
 *   Other arguments as for chunkattn_queue_step.
 */
int chunkattn_full(chunkattn_ctx *ctx, const void *q, const void *k, const void *v, void *out,
                   int batch, int lq, int lkv, long long kv_batch_stride, int heads,
                   int head_dim, float scale, int dtype, void *hip_stream);

/*
 * Argument checks of chunkattn_queue_step / chunkattn_full without a device:
 * the same validation those calls perform before launching.  Pointers are not
 * dereferenced.  The explanation of a failure is in chunkattn_last_error(NULL).
 */
int chunkattn_validate_queue_step(const void *q, const void *k, const void *v,
                                  const void *kv_cache, const void *out, int chunk_len,
                                  int n_chunks, int heads, int head_dim, float scale,
                                  int dtype);
int chunkattn_validate_full(const void *q, const void *k, const void *v, const void *out,
                            int batch, int lq, int lkv, long long kv_batch_stride, int heads,
                            int head_dim, float scale, int dtype);
int chunkattn_validate_window_step(const void *q, const void *k, const void *v,
                                   const void *kv_cache, const void *out, int chunk_len,
                                   int n_chunks, int heads, int head_dim, float scale,
                                   int dtype);
int chunkattn_validate_ring_step(const void *q_ring, const void *k_ring, const void *v_ring,
                                 const void *out_ring, int slots, int tail_slot, int n_live,
                                 int chunk_len, int heads, int head_dim, float scale,
                                 int dtype);

/* Static description of a status code. */
const char *chunkattn_status_string(int status);

/*
 * Explanation of the last failing call on this context, or of the last failing
 * validate call on this thread when ctx is NULL.  Empty string if none.  The
 * pointer stays valid until the next call on the same context/thread.
 */
const char *chunkattn_last_error(const chunkattn_ctx *ctx);

/*
 * The integer work plan of a queue step, without a device: one record of 7
 * ints per workgroup, in launch order (workgroup id 0, 1, ...):
 *   (chunk, head, q_row0, q_rows, pred_chunk, pred_rows, own_rows)
 * pred_chunk is c-1 when the chunk reads a predecessor (pred_rows = chunk_len),
 * else -1 (pred_rows = 0).  n_xcd is the number of accelerator dies the
 * workgroups are spread over (8 on MI355X; 1 disables the die-aware order);
 * block_rows is the work-item size (128, 256 or 384; 0 = chunkattn_block_rows()).
 * Writes at most `cap` records to `items` (may be NULL when cap is 0) and the
 * total count to *n_items.
 */
int chunkattn_plan_debug(int chunk_len, int n_chunks, int heads, int n_xcd, int block_rows,
                         int *items, long long cap, long long *n_items);

/*
 * The work plan of a window step, as chunkattn_plan_debug: the first field is
 * the window c; q_row0/q_rows index window c's 2 * chunk_len query rows (rows
 * >= chunk_len are chunk c+1's); own_rows is 2 * chunk_len (chunk_len for the
 * last window), read from chunk c onwards.
 */
int chunkattn_window_plan_debug(int chunk_len, int n_chunks, int heads, int n_xcd,
                                int block_rows, int *items, long long cap, long long *n_items);

/*
 * The same plan as decoded on the device by the attention kernel's own decode
 * routine: writes n_items * 7 ints to device memory `dev_items` on hip_stream,
 * using the context's die count and its work-item size for bf16, head_dim-128
 * calls (chunkattn_ctx_block_rows).  For bit-exact tests of the device decode.
 */
int chunkattn_plan_device(chunkattn_ctx *ctx, int chunk_len, int n_chunks, int heads,
                          int *dev_items, long long cap, void *hip_stream);

/* Number of accelerator dies (XCDs) the context uses for its launch order. */
int chunkattn_ctx_xcd_count(const chunkattn_ctx *ctx);

/*
 * Matrix-core rate probe, a measurement aid beside the attention path (it
 * computes nothing of the method): the dense bf16 rate the device sustains
 * under its own clock and power limit, against which the attention kernels'
 * throughput can be stated besides the rate quoted at 2.4 GHz.  One launch on
 * hip_stream: one workgroup of 8 waves per CU; every wave loads four operand
 * pairs (A, B) of the 16x16x32 bf16 matrix instruction and runs `iters`
 * rounds of 8 independent such instructions (accumulator a adds A_{a%4} B_{a%4}).
 *
 *   operands  device, 64 lanes x 32 words (pairs of bf16): lane l's words
 *             8s..8s+3 are its A fragment of pair s (row l % 16 of A, columns
 *             8*(l/16) .. +7), words 8s+4..8s+7 its B fragment (column l % 16
 *             of B, rows 8*(l/16) .. +7); the same for every wave.
 *   iters     rounds, 1 .. 2^19 (so that with entries in {-1, 0, 1} every
 *             accumulator stays an exact integer in fp32).
 *   out       device, n_workgroups * 8 waves * 8 accumulators * 64 lanes * 4
 *             floats: lane l's 4 values of accumulator a are rows
 *             4*(l/16) .. +3, column l % 16, of iters * A_{a%4} B_{a%4}.
 *   n_workgroups_out  receives the launch's workgroup count (the context's CU
 *             count), so out must hold chunkattn_ctx_cu_count(ctx) * 16384
 *             floats.
 *   flops_out receives the launch's FLOP count (2 per multiply-add).
 * Errors: CHUNKATTN_EINVAL for NULL or unaligned pointers or iters out of
 * range, CHUNKATTN_ELAUNCH if the launch fails.
 */
int chunkattn_mfma_probe(chunkattn_ctx *ctx, const void *operands, long long iters, void *out,
                         int *n_workgroups_out, double *flops_out, void *hip_stream);

/* Number of compute units of the context's device. */
int chunkattn_ctx_cu_count(const chunkattn_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKATTN_H */
