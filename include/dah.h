/*
 * dah.h -- C ABI of the Qwen3-0.6B decode-attention block on AMD MI355X (gfx950).
 *
 * One decode step of one attention layer, as the "Qwen3-0.6B" Model Spec page
 * defines it in its "Compute-graph nodes" table:
 *
 *   attn.qk_norm  y = x / sqrt(sum_j x_j^2 / 128 + eps) * w, per head, one gain
 *                 vector shared by all 16 query heads and one by all 8 key heads
 *                 (also the nnterp qwen3 page, "The Notes")
 *   attn.rope     pairs (i, i+64), i < 64, rotated by pos * theta^(-2i/128)
 *   attn.core     decodeGQA: o[b,h] = sum_{s < seq_lens[b]}
 *                   softmax_s(<q[b,h], k[b,s,h/2]> / sqrt(128)) * v[b,s,h/2]
 *
 * plus the write of the new token's key and value into a paged KV cache with
 * page size 16 (shape domain in "At a glance"; the "Supported models" page,
 * "What every spec covers", states decode attention over seq_lens[b] cached
 * positions).
 *
 * Fixed sizes (spec constants): 16 query heads, 8 KV heads, head dim 128,
 * page size 16.  Query head h reads KV head h / 2.  The *_ex calls (and
 * chunk_attn_step, the projections and the layer) also take the family's
 * other head counts -- 32, 40 or 64 query heads over the same 8 KV heads,
 * query head h reading KV head h / (H / 8).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked [device] are GPU global-memory pointers; tensors are dense
 *    and row-major in the order given.  The caller owns every buffer; the
 *    library never allocates, frees or synchronises.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *    stream).  Results are valid once that stream has reached the call.
 *  - The return value is a dah_status.  Nothing throws or aborts.  Argument
 *    problems visible on the host return DAH_ERR_* before anything is
 *    launched; a failed launch returns DAH_ERR_HIP.  dah_last_error() gives a
 *    one-line description of the last non-OK return on the calling thread.
 *  - Device-resident values cannot be checked without a synchronisation, so
 *    they are preconditions, with a defined fault-free result when violated:
 *      seq_lens[b] <= 0               o[b] = 0, nothing appended, q_out[b] is
 *                                     the normed query rotated at pos 0
 *      seq_lens[b] > max_seq_len, or > max_pages_per_seq * 16
 *                                     o[b] = NaN, nothing appended for b
 *      a needed block_table entry outside [0, num_pages)
 *                                     o[b] = NaN; nothing is read or written
 *                                     through that entry (the new token is
 *                                     still stored when its own page id is
 *                                     in the pool)
 *    The new token's page must not be shared with another sequence.
 *
 * KV cache layout
 * ---------------
 *  k_cache and v_cache are pools of pages, each [num_pages][8][16][128]
 *  = (physical page, KV head, slot, dim), elements float32 (DAH_F32) or
 *  bfloat16 (DAH_BF16).  One (page, KV head) tile of 16 positions is
 *  contiguous (4 KiB in bfloat16).  block_table is int32
 *  [B][max_pages_per_seq]: block_table[b][j] is the physical page of logical
 *  page j of sequence b, so position s of sequence b lives at
 *  (block_table[b][s / 16], slot s % 16).  Only the first
 *  ceil(seq_lens[b] / 16) entries of a row are read.
 *
 *  Stores into a bfloat16 cache round float32 to nearest, ties to even.
 *  All arithmetic is float32; RoPE angles are formed and reduced in float64.
 */
#ifndef DAH_H
#define DAH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DAH_NUM_HEADS 16
#define DAH_NUM_KV_HEADS 8
#define DAH_HEAD_DIM 128
#define DAH_PAGE_SIZE 16

typedef enum {
  DAH_F32 = 0,  /* float32 cache */
  DAH_BF16 = 1  /* bfloat16 cache */
} dah_dtype;

typedef enum {
  DAH_OK = 0,
  DAH_ERR_NULL = 1,      /* a required pointer is NULL */
  DAH_ERR_SHAPE = 2,     /* a size is out of range or sizes disagree */
  DAH_ERR_DTYPE = 3,     /* unknown cache dtype */
  DAH_ERR_ALIGN = 4,     /* a pointer lacks the alignment stated below */
  DAH_ERR_WORKSPACE = 5, /* workspace missing or smaller than dah_workspace_bytes */
  DAH_ERR_HIP = 6        /* the HIP runtime reported an error (no device, launch failure) */
} dah_status;

/*
 * qk_norm_rope_append -- nodes attn.qk_norm and attn.rope of the
 * "Qwen3-0.6B" Model Spec page ("Compute-graph nodes"; tensors in "Tensors of
 * the main nodes"), followed by the store of the new token into the cache.
 *
 * For every sequence b, with pos = seq_lens[b] - 1 (seq_lens counts the new
 * token):
 *   q_out[b,h] = rope(qk_norm(q[b,h], q_gain), pos)          h < 16
 *   k_cache at (block_table[b][pos/16], g, pos%16) = rope(qk_norm(k_new[b,g], k_gain), pos)
 *   v_cache at the same place                      = v_new[b,g]  (no norm)
 *
 *   q, q_out     [device] float32 [B][16][128], 16-byte aligned; q_out may equal q
 *   k_new, v_new [device] float32 [B][8][128], 16-byte aligned
 *   q_gain, k_gain [device] float32 [128]
 *   eps          RMSNorm epsilon (1e-6 for Qwen3-0.6B), added to the mean square
 *   rope_theta   RoPE base (1e6 for Qwen3-0.6B)
 *   k_cache, v_cache [device] pools as described above, 16-byte aligned
 *   cache_dtype  DAH_F32 or DAH_BF16
 *   num_pages    pages in each pool (>= 1)
 *   block_table  [device] int32 [B][max_pages_per_seq]
 *   seq_lens     [device] int32 [B]
 *   B            sequences (>= 1)
 */
int qk_norm_rope_append(const float* q, const float* k_new, const float* v_new,
                        const float* q_gain, const float* k_gain, float eps, float rope_theta,
                        void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                        const int32_t* block_table, int max_pages_per_seq,
                        const int32_t* seq_lens, int B, float* q_out, void* stream);

/*
 * paged_decode_gqa -- node attn.core (decodeGQA) of the "Qwen3-0.6B" Model
 * Spec page ("Compute-graph nodes"), over the paged cache:
 *
 *   o[b,h] = sum_{s < seq_lens[b]} softmax_s(<q[b,h], K[b,s,h/2]> / sqrt(128)) V[b,s,h/2]
 *
 * computed as flash decoding: the positions are cut into ranges (see
 * dah_plan_decode) whose partial (max, sum, weighted V) are merged with a
 * log-sum-exp combine.  The "Supported models" page ("Facts proved about the
 * specs": flashAttn_eq, softmax_shift) states that this equals the spec's
 * attention for any partition.  One launch, plus one for the merge when a
 * sequence is cut.
 *
 *   q            [device] float32 [B][16][128], already normed and roped, 16-byte aligned
 *   k_cache, v_cache [device] pools, 16-byte aligned; cache_dtype DAH_F32 or DAH_BF16
 *   num_pages, block_table, max_pages_per_seq, seq_lens, B  as above
 *   max_seq_len  host-side bound on every seq_lens[b] (>= 1, <= max_pages_per_seq*16);
 *                the planner uses it
 *   num_splits   0 = let the planner choose; 1 = one workgroup per sequence;
 *                n > 1 = every sequence in at most n equal splits (the planner
 *                may use fewer so that no split is empty)
 *   o            [device] float32 [B][16][128], 16-byte aligned
 *   workspace    [device] scratch of at least
 *                dah_workspace_bytes(B, max_seq_len, num_splits) bytes,
 *                256-byte aligned; may be NULL when that size is 0.  Its
 *                contents need no initialisation and are garbage afterwards.
 */
int paged_decode_gqa(const float* q, const void* k_cache, const void* v_cache, int cache_dtype,
                     int64_t num_pages, const int32_t* block_table, int max_pages_per_seq,
                     const int32_t* seq_lens, int B, int max_seq_len, int num_splits,
                     float* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * decode_attn_step -- the whole decode-attention block for one layer: the
 * result of qk_norm_rope_append followed by paged_decode_gqa on q_out, in one
 * kernel launch (plus the merge when a sequence is cut): every decode
 * workgroup norms and rotates its own query heads, and the workgroup that
 * holds a sequence's last page norms, rotates and stores the new key and
 * value and attends to them.  Arguments are those of the two calls, except
 * that q_out may be NULL: the step then writes o and the cache only (the
 * pointer checks of q_out apply to q instead).  q_out may equal q (in place
 * with a cut sequence, the call makes the two launches instead).
 */
int decode_attn_step(const float* q, const float* k_new, const float* v_new,
                     const float* q_gain, const float* k_gain, float eps, float rope_theta,
                     void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                     const int32_t* block_table, int max_pages_per_seq,
                     const int32_t* seq_lens, int B, int max_seq_len, int num_splits,
                     float* q_out, float* o, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * dah_plan_decode -- how paged_decode_gqa / decode_attn_step will cut the work
 * on a device with num_cus compute units (host-only, no device access).
 *
 *   DAH_PLAN_PER_SEQUENCE  one workgroup per sequence (8 waves, one per KV head);
 *                          chosen when the batch alone fills the device and no
 *                          sequence exceeds 128 pages
 *   DAH_PLAN_BALANCED      the batch's pages, in sequence order, cut into
 *                          `workgroups` equal ranges regardless of sequence
 *                          boundaries; sequences cut by a range boundary are
 *                          merged by a log-sum-exp combine (flashAttn_eq on the
 *                          "Supported models" page licenses any partition)
 *   DAH_PLAN_SPLIT         every sequence cut into `splits` ranges of
 *                          `pages_per_split` pages (num_splits > 1 asks for this;
 *                          also the fallback for batches over 4096 sequences)
 *
 * num_splits: 0 = automatic, 1 = per sequence, n > 1 = at most n splits.
 * The kernel (dah_decode_kernel below): the matrix-core form for a bfloat16
 * cache except under fixed splits at 2 query heads per KV head; the
 * environment variable DAH_DECODE_KERNEL=valu or =mfma, read once per
 * process, overrides that where the other form is built (VALU: any float32
 * cache, bfloat16 at 2 query heads per KV head; matrix cores: bfloat16) -- a
 * measurement aid, reported here as well as used by the calls.  Likewise
 * DAH_DECODE_PLAN=per_sequence, balanced or split replaces the automatic
 * layout (num_splits 0) where that layout applies.
 * Returns a dah_status.
 */
typedef enum {
  DAH_PLAN_PER_SEQUENCE = 0,
  DAH_PLAN_SPLIT = 1,
  DAH_PLAN_BALANCED = 2
} dah_plan_mode;

typedef enum {
  DAH_KERNEL_VALU = 0,  /* dot products on the vector ALUs (any cache dtype) */
  DAH_KERNEL_MFMA = 1   /* both products on the matrix cores (bfloat16 cache) */
} dah_decode_kernel;

typedef struct {
  int mode;               /* dah_plan_mode */
  int splits;             /* splits per sequence (PER_SEQUENCE: 1; BALANCED: 0) */
  int pages_per_split;    /* pages per split (PER_SEQUENCE: the longest sequence; BALANCED: 0) */
  int workgroups;         /* workgroups of the decode launch */
  size_t workspace_bytes; /* workspace the call needs */
  int kernel;             /* dah_decode_kernel: MFMA for a bfloat16 cache with 4+ query heads
                             per KV head, or with 2 unless mode is DAH_PLAN_SPLIT */
} dah_decode_plan;

/* For 16 query heads and a bfloat16 cache (the kernel field); the cut is the same for float32. */
int dah_plan_decode(int B, int max_seq_len, int num_splits, int num_cus, dah_decode_plan* out);

/*
 * dah_workspace_bytes -- workspace paged_decode_gqa and decode_attn_step need
 * on the current device for these arguments (0 when one split suffices).
 * Returns 0 as well for invalid arguments; the entry points then report the
 * problem.  Queries the current device's compute-unit count once per device.
 */
size_t dah_workspace_bytes(int B, int max_seq_len, int num_splits);

/* dah_workspace_bytes_for -- the same for an explicit compute-unit count (no device query). */
size_t dah_workspace_bytes_for(int B, int max_seq_len, int num_splits, int num_cus);

/*
 * The Qwen3 family's other group sizes (nnterp qwen3 page, "Grouped-query
 * attention, with 128-wide heads on every size": 32 query heads for 4B and
 * 8B, 40 for 14B, 64 for 32B, all over 8 KV heads of 128 dims; "What loads as
 * this family": RoPE base 5e6 for the 4B-2507 pair, which is the rope_theta
 * argument).  The *_ex calls are the calls above with the query-
 * head count num_heads in {16, 32, 40, 64} after B: q, q_out and o become
 * [B][num_heads][128], query head h reads KV head h / (num_heads / 8), and
 * the workspace's partial results scale with num_heads.  Everything else -- the cache pools,
 * block table, sequence lengths, statuses -- is as above; num_heads outside
 * the set returns DAH_ERR_SHAPE.  The calls above are these with num_heads = 16.
 */
int qk_norm_rope_append_ex(const float* q, const float* k_new, const float* v_new,
                           const float* q_gain, const float* k_gain, float eps, float rope_theta,
                           void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                           const int32_t* block_table, int max_pages_per_seq,
                           const int32_t* seq_lens, int B, int num_heads, float* q_out,
                           void* stream);

int paged_decode_gqa_ex(const float* q, const void* k_cache, const void* v_cache,
                        int cache_dtype, int64_t num_pages, const int32_t* block_table,
                        int max_pages_per_seq, const int32_t* seq_lens, int B, int num_heads,
                        int max_seq_len, int num_splits, float* o, void* workspace,
                        size_t workspace_bytes, void* stream);

int decode_attn_step_ex(const float* q, const float* k_new, const float* v_new,
                        const float* q_gain, const float* k_gain, float eps, float rope_theta,
                        void* k_cache, void* v_cache, int cache_dtype, int64_t num_pages,
                        const int32_t* block_table, int max_pages_per_seq,
                        const int32_t* seq_lens, int B, int num_heads, int max_seq_len,
                        int num_splits, float* q_out, float* o, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * decode_attn_step_noalloc -- decode_attn_step_ex without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split partials live in a static device array of DAH_SCRATCH_BYTES (16 MiB)
 * that the library holds on each GPU it runs on until the process ends; the
 * call allocates nothing and calls no allocating routine.  Arguments and
 * results are those of decode_attn_step_ex (q_out may be NULL).
 *
 * A plan whose workspace (dah_workspace_bytes_ex) exceeds DAH_SCRATCH_BYTES
 * returns DAH_ERR_WORKSPACE before anything is launched.  At 16 query heads
 * that leaves room for the balanced plan up to 1,760 sequences and for
 * B * splits <= 2,016 under fixed splits (a quarter of that at 64 heads);
 * one workgroup per sequence needs none.  Every call on one GPU shares
 * that GPU's array, which keeps the last call's contents (no call needs it
 * cleared): calls that overlap on one GPU -- on different streams, or on one
 * stream while another thread also calls -- race on it.
 */
#define DAH_SCRATCH_BYTES (16u << 20)
int decode_attn_step_noalloc(const float* q, const float* k_new, const float* v_new,
                             const float* q_gain, const float* k_gain, float eps,
                             float rope_theta, void* k_cache, void* v_cache, int cache_dtype,
                             int64_t num_pages, const int32_t* block_table,
                             int max_pages_per_seq, const int32_t* seq_lens, int B,
                             int num_heads, int max_seq_len, int num_splits, float* q_out,
                             float* o, void* stream);

/*
 * The planner and workspace size for num_heads query heads and a cache of
 * cache_dtype: with a bfloat16 cache and 32 or more heads the decode runs on
 * the matrix cores, and the balanced plan starts at 32 sequences instead of
 * 64.  dah_plan_decode_ex returns DAH_ERR_DTYPE for an unknown dtype;
 * dah_workspace_bytes_ex returns 0 for invalid arguments.
 */
int dah_plan_decode_ex(int B, int num_heads, int cache_dtype, int max_seq_len, int num_splits,
                       int num_cus, dah_decode_plan* out);

size_t dah_workspace_bytes_ex(int B, int num_heads, int cache_dtype, int max_seq_len,
                              int num_splits);

/*
 * chunk_attn_step -- several new tokens per sequence (chunked prefill, or
 * verification of drafted tokens): for every sequence b with chunk tokens
 * t = cu_tokens[b] .. cu_tokens[b+1]-1 (n_b = cu_tokens[b+1] - cu_tokens[b],
 * 0 allowed), token i of the chunk sits at position seq_lens[b] - n_b + i
 * (seq_lens counts the cache after the chunk).  Each token is normed and
 * rotated at its position and its key and value appended as in
 * qk_norm_rope_append; then every token attends (decodeGQA over positions
 * 0 .. its own) causally -- the Model Spec page's shape domain allows
 * T in [1, 40,960] new tokens, and forward_causal ("Supported models" page)
 * states that later tokens cannot change earlier outputs.
 *
 *   q, q_out     [device] float32 [total_tokens][H][128]; q_out may equal q
 *   k_new, v_new [device] float32 [total_tokens][8][128]
 *   o            [device] float32 [total_tokens][H][128]
 *   cu_tokens    [device] int32 [B+1], non-decreasing, cu_tokens[B] = total_tokens
 *   max_chunk    host bound on every n_b (1 .. total_tokens); the grids are sized by it
 *   max_seq_len  host bound on every seq_lens[b] (<= max_pages_per_seq * 16)
 *   num_heads    16, 32, 40 or 64
 *   other arguments as in decode_attn_step (cache DAH_BF16 or DAH_F32).
 *
 * Two launches (append, attention), no workspace.  A bfloat16 cache runs on
 * the matrix cores, each cached page read once per tile of 16/G tokens (or
 * once per 4 such tiles, shared through LDS, for longer chunks: there q
 * enters the score product as two bfloat16 terms, to a relative 2^-18 like
 * the softmax weights, where the one-tile kernel and the decode use three);
 * a float32
 * cache runs every token as its own decode on the VALU path (each token
 * reads its prefix: meant for verification-sized chunks and strict-parity
 * runs).  A sequence with
 * seq_lens[b] < n_b, seq_lens[b] > max_seq_len or n_b > max_chunk gets NaN
 * outputs and no append; a page id outside the pool gives NaN for the tokens
 * that read it.
 */
int chunk_attn_step(const float* q, const float* k_new, const float* v_new, const float* q_gain,
                    const float* k_gain, float eps, float rope_theta, void* k_cache,
                    void* v_cache, int cache_dtype, int64_t num_pages,
                    const int32_t* block_table, int max_pages_per_seq, const int32_t* seq_lens,
                    const int32_t* cu_tokens, int B, int total_tokens, int max_chunk,
                    int max_seq_len, int num_heads, float* q_out, float* o, void* stream);

/*
 * The linear layers on either side of the block: attn.qkv_proj and
 * attn.o_proj of the "Qwen3-0.6B" Model Spec page ("Compute-graph nodes",
 * the `linear` rows: y[t,n] = sum_k x[t,k] w[n,k]), on the matrix cores.
 * Activations are float32, weights bfloat16 (the checkpoints' dtype, nnterp
 * qwen3 page, configuration table), outputs float32.  x enters the products
 * as two bfloat16 terms (2^-18 relative), accumulation is float32.
 *
 * dah_linear -- y [T][N] = x [T][K] . w^T, w [N][K] row-major (device
 *   pointers, 16-byte aligned).  T >= 1; N a multiple of 64; K a multiple of
 *   256.  Returns DAH_ERR_NULL / _SHAPE / _ALIGN before any launch.
 *
 * attn_qkv_proj -- x [T][hidden] times w_qkv [H*128 + 2048][hidden], whose
 *   rows are q_proj (H*128 rows), k_proj (1024) and v_proj (1024) stacked;
 *   the outputs go to q [T][H][128], k [T][8][128], v [T][8][128] -- the
 *   layouts decode_attn_step[_ex] takes as q, k_new, v_new.  H = num_heads
 *   in {16, 32, 40, 64}; hidden a multiple of 256 (1024 for Qwen3-0.6B).
 *
 * attn_o_proj -- o [T][H][128] (heads side by side, as decode_attn_step
 *   writes it) times w_o [hidden][H*128] -> y [T][hidden]; hidden a multiple
 *   of 64.
 *
 * None of them allocates or synchronises; stream as for the other calls.
 */
int dah_linear(const float* x, const void* w, int T, int N, int K, float* y, void* stream);

int attn_qkv_proj(const float* x, const void* w_qkv, int T, int hidden, int num_heads, float* q,
                  float* k, float* v, void* stream);

int attn_o_proj(const float* o, const void* w_o, int T, int num_heads, int hidden, float* y,
                void* stream);

/*
 * dah_linear_residual -- y = x . w^T + residual (shapes as dah_linear;
 *   residual [T][N] float32, 16-byte aligned, may equal y): the residual
 *   adds of the decoder layer (attn_residual, mlp_residual) folded into the
 *   product's store.
 */
int dah_linear_residual(const float* x, const void* w, const float* residual, int T, int N,
                        int K, float* y, void* stream);

/*
 * A product with the RMSNorm before it folded in (the decoder layer's
 * input_norm / post_attn_norm + linear rows of the "Qwen3-0.6B" Model Spec
 * page, "Compute-graph nodes"):
 *
 * dah_rmsnorm_linear -- y = rmsnorm(x) . w^T, rmsnorm(x)[t][k] =
 *   x[t][k] / sqrt(sum_j x[t][j]^2 / K + eps) * x_gain[k]; shapes as
 *   dah_linear, x_gain [K] float32 (16-byte aligned), eps >= 0.  The sum of
 *   squares is accumulated as x streams through the product and 1/rms scales
 *   each output row; the normed rows are never stored.  Errors as
 *   dah_linear (and DAH_ERR_NULL for a NULL gain).
 */
int dah_rmsnorm_linear(const float* x, const float* x_gain, float eps, const void* w, int T,
                       int N, int K, float* y, void* stream);

/*
 * dah_rmsnorm_swiglu -- the MLP's first half in one launch (the
 * post_attn_norm, mlp.gate_up and mlp.act rows of the "Qwen3-0.6B" Model
 * Spec page, "Compute-graph nodes"):
 *   h = rmsnorm(x) as dah_rmsnorm_linear (x as stored when x_gain is NULL),
 *   [gate | up] = h . w_gate_up^T, act[t][j] = silu(gate[t][j]) * up[t][j],
 *   silu(z) = z / (1 + e^-z), j < inter.
 *   x [T][K] float32; w_gate_up [2 inter][K] bfloat16, the gate rows then
 *   the up rows (the checkpoint's order); act [T][inter] float32; inter a
 *   positive multiple of 32, K of 256; 16-byte alignment.  Each product tile
 *   holds gate and up columns of the same j side by side, so the activation
 *   is applied as the tile is stored and [gate | up] is never written.
 *   Errors as dah_rmsnorm_linear.
 */
int dah_rmsnorm_swiglu(const float* x, const float* x_gain, float eps, const void* w_gate_up,
                       int T, int inter, int K, float* act, void* stream);

/*
 * Products that split k over workgroups (the o_proj and down rows of the
 * "Qwen3-0.6B" Model Spec page, "Compute-graph nodes": K = H*128 or 3072
 * against N = 1024 outputs gives few output tiles for the chip).  Each
 * workgroup multiplies one output tile over one of 4 or 8 equal k slices
 * into a float32 partial product in the caller's workspace; a second launch
 * adds the slices in slice order and the residual.  The sum is the same
 * product up to float32 rounding order.
 *
 * dah_linear_workspace_bytes -- host only: the workspace dah_linear_ws needs
 *   for a T x N x K product (k slices x T x N x 4 bytes), 0 when it does not
 *   split k (K < 2048) or the shape is invalid.
 *
 * dah_linear_ws -- y = x . w^T (+ residual when residual is not NULL); shapes,
 *   alignment and errors as dah_linear_residual, and workspace (device,
 *   256-byte aligned, may be NULL when dah_linear_workspace_bytes is 0) of
 *   workspace_bytes >= dah_linear_workspace_bytes(T, N, K), else
 *   DAH_ERR_WORKSPACE before any launch.  residual may equal y; the
 *   workspace must not overlap x, w, residual or y.  Its contents on entry
 *   do not matter and are left undefined.
 *
 * attn_o_proj_ws -- attn_o_proj through dah_linear_ws (K = num_heads * 128).
 *
 * dah_linear_ws_kernel -- host only: the kernel dah_linear_ws launches (ids
 *   as dah_linear_kernel) and, in *k_slices (may be NULL), its k slices (1 =
 *   unsplit); -1 for an invalid shape.
 */
size_t dah_linear_workspace_bytes(int T, int N, int K);

int dah_linear_ws(const float* x, const void* w, const float* residual, int T, int N, int K,
                  float* y, void* workspace, size_t workspace_bytes, void* stream);

int attn_o_proj_ws(const float* o, const void* w_o, int T, int num_heads, int hidden, float* y,
                   void* workspace, size_t workspace_bytes, void* stream);

int dah_linear_ws_kernel(int T, int N, int K, int* k_slices);

/*
 * dah_linear_kernel -- host only, no device call: which kernel dah_linear
 *   (and the projections built on it) launches for a T x N x K product:
 *   0 = the split-k kernel (decode's few rows), 1..5 = the LDS-tiled kernel
 *   with tiles 64x128, 64x64, 32x64, 32x32, 32x32 with 256-wide k chunks;
 *   -1 if the shape is invalid.  For tests and benchmarks.
 */
int dah_linear_kernel(int T, int N, int K);

/*
 * dah_rmsnorm -- rows of a hidden-size RMSNorm (the input_norm,
 *   post_attn_norm and final_norm rows of the Model Spec page:
 *   y = x / sqrt(sum x^2 / H + eps) * w, H = width): x, y [T][width]
 *   float32 (may be the same), w [width] float32; width a multiple of 4;
 *   16-byte alignment.
 *
 * dah_silu_mul -- mlp.act: act[t][i] = silu(g[t][i]) * g[t][inter + i],
 *   silu(z) = z / (1 + e^-z); gate_up [T][2 inter], act [T][inter] float32.
 */
int dah_rmsnorm(const float* x, const float* w, float eps, int T, int width, float* y,
                void* stream);

int dah_silu_mul(const float* gate_up, int T, int inter, float* act, void* stream);

/*
 * decoder_layer_step -- one decoder layer's decode step (the per-layer rows
 * of the Model Spec page's "Compute-graph nodes", in order): input_norm,
 * attn.qkv_proj, the attention step (decode_attn_step_ex), attn.o_proj plus
 * the attention residual, post_attn_norm, mlp.gate_up, mlp.act and mlp.down
 * plus the MLP residual.
 *
 *   x, y         [device] float32 [B][hidden] (the residual stream in and
 *                out; y may equal x)
 *   w            the layer's weights (pointers to device memory, below)
 *   hidden, inter  model width and MLP width, multiples of 256 (1024 and
 *                3072 for Qwen3-0.6B)
 *   num_heads, eps, rope_theta, the cache, block table, seq_lens, B,
 *   max_seq_len, num_splits   as for decode_attn_step_ex
 *   workspace    [device] at least dah_layer_workspace_bytes(...) bytes,
 *                256-byte aligned (the intermediates, then one region
 *                shared by the attention's workspace and the k-slice
 *                partials of o_proj and down, which run through
 *                dah_linear_ws); contents need no initialisation.
 *
 * Five to eight launches in order on `stream`: qkv_proj (input_norm folded
 * in), the attention step (plus its merge when a sequence is cut over
 * workgroups), o_proj (plus its slice reduce when k is split), gate_up with
 * post_attn_norm and mlp.act folded in (dah_rmsnorm_swiglu), down (plus its
 * slice reduce).  The attention's arguments are checked before the first.
 */
typedef struct {
  const float* w_in;       /* input_norm gain [hidden], float32 */
  const void* w_qkv;       /* bfloat16 [(H + 16) * 128][hidden]: q_proj, k_proj, v_proj rows */
  const float* q_gain;     /* q_norm gain [128] */
  const float* k_gain;     /* k_norm gain [128] */
  const void* w_o;         /* bfloat16 [hidden][H * 128] */
  const float* w_post;     /* post_attn_norm gain [hidden] */
  const void* w_gate_up;   /* bfloat16 [2 * inter][hidden]: gate rows, then up rows */
  const void* w_down;      /* bfloat16 [hidden][inter] */
} dah_layer_weights;

size_t dah_layer_workspace_bytes(int B, int hidden, int inter, int num_heads, int cache_dtype,
                                 int max_seq_len, int num_splits);

int decoder_layer_step(const float* x, const dah_layer_weights* w, int hidden, int inter,
                       int num_heads, float eps, float rope_theta, void* k_cache, void* v_cache,
                       int cache_dtype, int64_t num_pages, const int32_t* block_table,
                       int max_pages_per_seq, const int32_t* seq_lens, int B, int max_seq_len,
                       int num_splits, float* y, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Static name of a dah_status value ("DAH_OK", ...); "unknown status" otherwise. */
const char* dah_status_string(int status);

/* Detail of the last non-OK return on this thread ("" if none).  Valid until the next call. */
const char* dah_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DAH_H */
