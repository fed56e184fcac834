/*
 * mdm_sparse.h - C ABI of the sparse masked-diffusion sampling step (HIP, gfx950).
 *
 * One sampling step of Sparse-LaViDa (arXiv 2512.14008) processes only a small
 * query set: the tokens decoded at the previous step (they enter the KV cache
 * now), the masked positions chosen for decoding at this step, and R register
 * tokens placed after the end of the sequence; logits are produced only for
 * the decoded subset (papernotes.org reading notes, page 1: overall framework,
 * key designs 1-3 and the worked example = the paper's Figure 3; paperlayer.ai
 * summary, section 3.2).
 *
 * The model behind these calls is one attention layer whose query/key/value
 * rows are looked up by token id in folded tables (embedding times projection),
 * rotated by RoPE at each row's explicit position id; h is the concatenation of
 * the head outputs and the logits are h W^T.  Token ids: 0..V-1 vocabulary,
 * V = the mask token, V+1..V+R the registers.  Positions are 0-indexed; the
 * registers sit at seq_len .. seq_len+R-1.
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    never allocates or frees device memory and keeps no pointer beyond the
 *    buffers registered at init.  It allocates only the host-side context.
 *  - Every compute call is an asynchronous enqueue on the context's stream and
 *    returns after validating its arguments on the host; results are valid
 *    once that stream has been synchronised.  On an argument, shape or
 *    capacity error nothing is enqueued; a launch failure (MDM_E_HIP) inside a
 *    call of several launches can leave its earlier launches enqueued.
 *  - "bf16" arrays hold bfloat16 bit patterns (uint16); "elem" means bf16 in
 *    MDM_BF16 precision and fp32 in MDM_FP32 precision.
 *  - A context is not thread-safe; use one context per stream.
 *  - Token ids and positions in device arrays are range-checked by the
 *    kernels: an out-of-range value is replaced by 0 for addressing and sets a
 *    sticky flag that mdm_device_status() reports as MDM_E_DEVICE.
 */
#ifndef MDM_SPARSE_H
#define MDM_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MDM_OK = 0,
  MDM_E_ARG = -1,          /* null pointer, bad enum or out-of-range scalar           */
  MDM_E_SHAPE = -2,        /* sizes inconsistent with the config or the buffers      */
  MDM_E_CAPACITY = -3,     /* more rows than the sequence (seq_len) can hold          */
  MDM_E_HIP = -4,          /* a HIP runtime call failed (see mdm_last_error)          */
  MDM_E_UNSUPPORTED = -5,  /* a shape this build does not implement                   */
  MDM_E_DEVICE = -6        /* a kernel met an out-of-range token id or position       */
} mdm_status;

typedef enum {
  MDM_BF16 = 0,            /* bf16 storage, bf16 MFMA with fp32 accumulation          */
  MDM_FP32 = 1             /* fp32 storage and arithmetic (validation mode)           */
} mdm_precision;

typedef enum {
  MDM_SELECT_ORDER = 0,       /* pre-generated order: unmask every candidate           */
  MDM_SELECT_CONFIDENCE = 1   /* unmask the n_select most confident candidates         */
} mdm_select_mode;

typedef struct mdm_ctx mdm_ctx;   /* opaque host-side context */

typedef struct {
  int32_t batch;          /* B independent sequences, same per-step counts           */
  int32_t n_heads;        /* H query heads                                            */
  int32_t n_kv_heads;     /* H_kv key/value heads; H % H_kv == 0; query head h uses   */
                          /* key/value head h / (H / H_kv)                            */
  int32_t head_dim;       /* d: 64 or 128                                             */
  int32_t vocab;          /* V                                                        */
  int32_t seq_len;        /* total length of the sequence (prompt + generated)       */
  int32_t n_registers;    /* R, 0..256                                                */
  int32_t max_decode;     /* upper bound on n_decode per step (sizes the workspace)  */
  int32_t precision;      /* mdm_precision                                            */
  int32_t accurate_conf;  /* bf16 only: nonzero splits h into bf16 hi + lo for the    */
                          /* vocab screening, so confidences are accurate enough to   */
                          /* rank; zero screens with bf16(h) (the argmax is exact     */
                          /* either way: see mdm_subset_logits_confidence)            */
  double rope_theta;      /* RoPE base (10000)                                        */
} mdm_config;

typedef struct {
  const void* tq;         /* elem [V+1+R][H*d]    folded query table, row = token id  */
  const void* tk;         /* elem [V+1+R][H_kv*d] folded key table                    */
  const void* tv;         /* elem [V+1+R][H_kv*d] folded value table                  */
  const void* w_vocab;    /* elem [V][H*d]        vocabulary head                     */
  void* k_cache;          /* elem [B][H_kv][slots][d]   RoPE'd keys, append order     */
  void* v_cache;          /* elem [B][H_kv][slots/64][d][64]  values, transposed in
                             64-slot tiles: slot s of dim d sits at
                             ((s/64)*d_head + d)*64 + s%64 within its (b, kv head) */
  int32_t* cache_pos;     /* [B][slots] position id of each cached slot               */
  int32_t* cache_tok;     /* [B][slots] token id of each cached slot                  */
  void* workspace;        /* scratch, at least mdm_workspace_bytes() bytes, 256-aligned */
  size_t workspace_bytes;
} mdm_buffers;

/* Slots per (sequence, key/value head) in the cache buffers: seq_len rounded up
 * to a multiple of 64.  Returns 0 for an invalid config. */
size_t mdm_cache_slots(const mdm_config* cfg);

/* Bytes of workspace the context needs (RoPE table, the key/query/value tables of
 * the mask token and the registers, the appended rows' queries, packed h,
 * partial results; bf16 with vocab >= 32768: a copy of w_vocab tiled for the
 * vocabulary screen, V rounded up to 512 rows x H*d x 2 bytes).  0 if invalid. */
size_t mdm_workspace_bytes(const mdm_config* cfg);

/* Bytes per element of tables, caches and the vocab head (2 or 4).  0 if invalid. */
size_t mdm_element_bytes(const mdm_config* cfg);

/* Create a context (page 3, section 3.2: the cache starts empty and the prompt
 * is prefetched into it by mdm_kv_append).  Validates cfg and the buffers,
 * builds the fp32 RoPE table (cos/sin of pos * base^(-2i/d) evaluated in double,
 * rounded to fp32) on the host and uploads it to the workspace, clears the
 * device error flag, builds in the workspace the rows every step reuses (bf16:
 * the RoPE'd keys and queries of the mask token at every position and of the
 * registers, and their values in the layout the attention tiles read; for
 * vocab >= 32768 a copy of w_vocab in 128-row x 64-column runs, which the
 * vocabulary screen streams), and computes the largest row norm of w_vocab
 * (for the decisions' error bound),
 * and synchronises the stream once.  The tables tq/tk/tv and w_vocab are read
 * here and by later calls, so they must hold their final contents before init
 * and not change while the context lives.  `stream` is a hipStream_t (NULL = the default
 * stream).  On success *ctx owns a host allocation released by
 * mdm_sparse_step_destroy. */
mdm_status mdm_sparse_step_init(mdm_ctx** ctx, const mdm_config* cfg, const mdm_buffers* buf,
                                void* stream);

/* Change the stream later calls enqueue on (e.g. a graph-capture stream). */
mdm_status mdm_set_stream(mdm_ctx* ctx, void* stream);

/* Append n rows to every sequence's KV cache (page 3, section 3.2: the prompt is
 * prefetched; the tokens decoded at step k-1 enter the cache before step k).
 * Row r of sequence b has token id tok[b*stride + r] and position pos[b*stride + r];
 * its key is Tk[id] rotated by RoPE at pos, its value Tv[id]; both are written
 * to slot len+r, with (pos, id) recorded in cache_pos / cache_tok.  The host
 * cache length becomes len + n.  stride 0 means n.  MDM_E_CAPACITY if
 * len + n > seq_len.  n == 0 is a no-op.  bf16 with n <= max_decode: the same
 * launch also writes the n rows' RoPE'd queries (every query head) into the
 * workspace, where the next mdm_step_attention takes them for its D rows. */
mdm_status mdm_kv_append(mdm_ctx* ctx, const int32_t* tok, const int32_t* pos, int64_t stride,
                         int32_t n);

/* Step attention under the step-causal mask (page 1, worked example = Figure 3;
 * page 1, key design 3).  The query set of every sequence is, in this order:
 *   n_new_cached rows D (token d_tok, position d_pos) - the rows the preceding
 *     mdm_kv_append committed, in the same order; they see the cache (which
 *     includes themselves); when that append wrote their queries (see
 *     mdm_kv_append) the kernel reads those, else it rotates them itself;
 *   n_decode rows C (the mask token at positions c_pos[b*c_stride + i]);
 *   R register rows (ids V+1.., positions seq_len..);
 * C and R rows see the cache plus all C and R rows.  Keys, values and queries
 * of the C and R rows come from the rows built at init (the mask token's key
 * depends only on its position); they are never written to the cache.  One
 * attention kernel launch, plus a small merge launch when the key range of a
 * (sequence, head) is split over several blocks.  Output
 * out[b][i][h*d + j] (fp32, [B][n_q][H*d], n_q = n_new_cached + n_decode + R) is
 * the attention output of row i, head h.  Strides of 0 mean compact.
 * MDM_E_CAPACITY if len + n_decode > seq_len; MDM_E_ARG if n_new_cached > len
 * or n_decode > max_decode (bf16 also requires max_decode <= 2048, checked at
 * init). */
mdm_status mdm_step_attention(mdm_ctx* ctx, const int32_t* d_tok, const int32_t* d_pos,
                              int64_t d_stride, int32_t n_new_cached, const int32_t* c_pos,
                              int64_t c_stride, int32_t n_decode, float* out);

/* Logits for the decoded subset only, with confidence and argmax (page 1, key
 * design 1: only the positions being decoded need logits; page 3, section 3.2).
 * Row c of sequence b is h[b*h_batch_stride + c*H*d .. +H*d) (fp32).  For every
 * row: token = the lowest index of the largest logit z = h W^T, conf = the
 * largest softmax probability (temperature 1).  All logits are first screened
 * (bf16 path: a bf16 MFMA product of bf16(h), or of its hi + lo split with
 * accurate_conf; fp32 path: fp32 products), keeping per 128-column tile the
 * maximum, the sum of exponentials and the three best entries.  The 8 best
 * entries are then re-scored exactly in fp32 from the fp32 h, and a bound on
 * the screen's error (Cauchy-Schwarz on h minus its screened copy, times the
 * largest vocabulary row norm, plus the accumulation error) proves that no
 * other column reaches the best exact logit; where it cannot, the kernel
 * re-scores every entry (or whole tile) that might, so the token is the argmax
 * of the fp32 logits over the whole vocabulary.  conf uses the screened
 * logits with the re-scored entries' terms exact.
 * conf, token: [B][n_decode].  logits_or_null: if non-NULL, receives the
 * screened logits [B][n_decode][V] (fp32). */
mdm_status mdm_subset_logits_confidence(mdm_ctx* ctx, const float* h, int64_t h_batch_stride,
                                        int32_t n_decode, float* conf, int32_t* token,
                                        float* logits_or_null);

/* Unmasking after a step (page 3, section 3.2).  Candidates i of sequence b:
 * position cand_pos[b*cand_stride + i], decided token token[b*n_cand + i],
 * confidence conf[b*n_cand + i].
 *   MDM_SELECT_ORDER: n_select must equal n_cand; all candidates are unmasked
 *     in the given order.
 *   MDM_SELECT_CONFIDENCE: the n_select candidates with the largest conf (ties:
 *     lower position first) are unmasked; they are listed in ascending
 *     position order, and the others (still masked) are written in ascending
 *     position order to rem_pos[b][n_cand - n_select] (may be NULL).
 * out_tok/out_pos [B][n_select] receive the unmasked tokens and positions (the
 * rows entering the cache at the next step); seq_tokens[b][pos] = token for
 * each unmasked position if seq_tokens is non-NULL ([B][seq_len]). */
mdm_status mdm_unmask_select(mdm_ctx* ctx, const int32_t* cand_pos, int64_t cand_stride,
                             const float* conf, const int32_t* token, int32_t n_cand,
                             int32_t n_select, int32_t mode, int32_t* out_tok, int32_t* out_pos,
                             int32_t* rem_pos, int32_t* seq_tokens);

/* One whole sampling step when the unmasking order is fixed beforehand (page 3,
 * section 3.2: image tokens are unmasked in a pre-generated order, so every
 * decoded position is unmasked), in two fewer launches than the separate
 * calls.  The results are those of the sequence
 *   mdm_step_attention(ctx, D rows, n_new_cached, c_pos, c_stride, n_decode, out);
 *   mdm_subset_logits_confidence(ctx, C rows of out, ..., n_decode, conf, token, logits_or_null);
 *   mdm_unmask_select(ctx, c_pos, c_stride, conf, token, n_decode, n_decode,
 *                     MDM_SELECT_ORDER, ..., seq_tokens);
 *   if (commit) mdm_kv_append(ctx, token, c_pos, ..., n_decode);
 * bit for bit: the attention also writes the bf16 split of the C rows'
 * outputs for the logits, the merge of the logits writes each decided token
 * at its position (seq_tokens[b][pos], if non-NULL), and with commit non-zero
 * the decided rows are appended (slot len + c for candidate c) with their
 * queries kept, so that they are the D rows (n_new_cached) of the next call.
 * Leave commit 0 on the last step of a generation.
 * n_new_cached: 0, or the row count of the preceding commit (this call's or
 * mdm_kv_append's) on this context, whose queries the context kept; their
 * token ids and positions are not needed.  out [B][n_q][H*d] fp32 (16-byte
 * aligned), conf/token [B][n_decode], logits_or_null as in
 * mdm_subset_logits_confidence.  Errors as in the four calls; MDM_E_ARG if
 * n_new_cached is not 0 or that row count; MDM_E_UNSUPPORTED for the fp32
 * precision or with upper layers attached (use the separate calls). */
mdm_status mdm_order_step(mdm_ctx* ctx, int32_t n_new_cached, const int32_t* c_pos, int64_t c_stride,
                          int32_t n_decode, int32_t commit, float* out, float* conf, int32_t* token,
                          int32_t* seq_tokens, float* logits_or_null);

/* Start a new generation: cache length 0 (the buffers are reused). */
mdm_status mdm_sparse_step_reset(mdm_ctx* ctx);

/* Current cache length (host bookkeeping), -1 for NULL. */
int32_t mdm_cache_len(const mdm_ctx* ctx);

/* Shorten the cache to its first new_len slots (page 1, ablation Table 6: the
 * prompt and the decoded tokens may be recomputed at every step instead of
 * being kept, so a caller appends them again and drops them after the step).
 * Host bookkeeping only: nothing is enqueued, and later appends overwrite the
 * dropped slots.  Unless new_len equals the current length, the queries kept
 * by the last append are dropped too (a later mdm_step_attention rotates its
 * D rows itself; mdm_order_step then needs n_new_cached == 0).  MDM_E_ARG if
 * new_len < 0 or new_len > the current length; MDM_E_UNSUPPORTED with upper
 * layers attached (their caches are not shortened). */
mdm_status mdm_cache_rewind(mdm_ctx* ctx, int32_t new_len);

/* Synchronise the stream, read and clear the kernels' sticky range-check flag.
 * MDM_E_DEVICE if any kernel met an out-of-range token id or position. */
mdm_status mdm_device_status(mdm_ctx* ctx);

/* Per-row certificate of the logits decisions (page 1, key design 1: the
 * decision is over the whole vocabulary).  With trace non-NULL (device, 16-byte
 * aligned, caller-owned, at least B*max_decode rows of 8 floats), every later
 * mdm_subset_logits_confidence / mdm_order_step writes for decided row m
 * (= b*n_decode + c) trace[m*8 ..]: {z1, i1, z2, i2, D, eps_s, eps_e, flags}:
 * z1 the exact fp32 logit of the decided token i1, z2/i2 the best exact logit
 * among the other re-scored columns, D an upper bound on the screened logit of
 * every column not re-scored, eps_s / eps_e the bounds on the screen's and the
 * re-score's error (so D + eps_s < z1 - eps_e proves the argmax), flags bit 0:
 * entries beyond the 8 candidates were re-scored, bit 1: whole tiles were,
 * bit 2: z1 - z2 <= 2 eps_e (a tie at fp32 precision), bit 3: the argmax is
 * proven.  i1, i2 and flags are int32 bit patterns.  NULL turns it off. */
mdm_status mdm_set_decision_trace(mdm_ctx* ctx, float* trace);

/* Synchronise the stream and read, then clear, the decision counters since the
 * previous read: out[0] rows that re-scored entries beyond the 8 candidates,
 * out[1] rows that re-scored whole tiles, out[2] rows whose two best exact
 * logits were within twice the re-score error bound. */
mdm_status mdm_decision_counts(mdm_ctx* ctx, int64_t* out);

/* ---- upper layers --------------------------------------------------------
 * A model of L >= 2 attention layers without W_o, MLP or norms: layer l >= 2
 * takes the previous layer's head outputs h_{l-1} of every query row and
 * projects them, [q | k | v] = h_{l-1} W_l^T, with q and k RoPE'd at the row's
 * position and all three rounded to bf16.  Each layer has its own cache; the
 * rows decoded at step k-1 enter every layer's cache at step k, which is what
 * makes the cache reuse of page 1 (overall framework: cached representations
 * are not polluted by the masked rows) load-bearing: layer l's cached keys
 * were computed from layer l-1 outputs of a D row, which saw only the cache.
 * bf16 precision only.  A step with L layers:
 *   mdm_kv_append(D); mdm_step_attention(...) -> h_1
 *   for l = 2..L: mdm_layer_project(l, h_{l-1}, ...); mdm_layer_attention(l, ...) -> h_l
 *   mdm_subset_logits_confidence(C rows of h_L)
 * Prefill: mdm_kv_append(prompt); mdm_step_attention(D = prompt, n_decode = 0)
 * -> h_1; then per upper layer mdm_layer_project(D = prompt) (and, below the
 * top layer, mdm_layer_attention) so that every layer caches the prompt. */
typedef struct {
  int32_t n_layers;        /* L, 2..16                                                   */
  const void* w_upper;     /* bf16 [L-1][(H + 2 H_kv) d][H d]: W_l of layers 2..L, rows  */
                           /* are the q heads, then the k heads, then the v heads        */
  void* k_cache_upper;     /* bf16 [L-1][B][H_kv][slots][d]   (layout of k_cache)        */
  void* v_cache_upper;     /* bf16 [L-1][B][H_kv][slots/64][d][64] (layout of v_cache)   */
  void* workspace;         /* mdm_upper_workspace_bytes() bytes, 256-byte aligned        */
  size_t workspace_bytes;
} mdm_upper_layers;

/* Bytes of the upper layers' workspace (packed h, the projected rows, the
 * queries and the C|R keys/values of one layer call); 0 if invalid or not bf16. */
size_t mdm_upper_workspace_bytes(const mdm_config* cfg);

/* Register the upper layers' weights, caches and workspace with ctx (caller-
 * owned, read and written by the calls below).  Resets their cache lengths.
 * MDM_E_UNSUPPORTED unless bf16; MDM_E_ARG for NULL, misaligned or n_layers
 * outside 2..16; MDM_E_SHAPE for a short workspace. */
mdm_status mdm_attach_upper_layers(mdm_ctx* ctx, const mdm_upper_layers* up);

/* Layer `layer` (2..L) projection of one step's query rows.  Row r of
 * sequence b is h_prev[b*h_batch_stride + r*H*d .. +H*d) (fp32) for r in
 * [0, n_q), n_q = n_new_cached + n_decode + R, rows in the order D | C | R
 * (the output layout of the attention calls; h_batch_stride 0 means n_q*H*d).
 * Positions: D rows d_pos[b*d_stride + r], C rows c_pos[b*c_stride + j],
 * registers seq_len + j.  The D rows' k and v are appended to the layer's
 * cache (its length grows by n_new_cached); the C|R rows' k and v and every
 * row's q stay in the workspace for the next mdm_layer_attention of this
 * layer.  h is split into bf16 hi + lo for the MFMA product, so q, k, v are
 * near-fp32 accurate before their bf16 rounding.  MDM_E_CAPACITY when the
 * layer's cache would pass seq_len or n_q > seq_len + R; MDM_E_ARG for
 * n_decode > max_decode and the usual pointer/stride errors. */
mdm_status mdm_layer_project(mdm_ctx* ctx, int32_t layer, const float* h_prev, int64_t h_batch_stride,
                             const int32_t* d_pos, int64_t d_stride, int32_t n_new_cached,
                             const int32_t* c_pos, int64_t c_stride, int32_t n_decode);

/* Layer `layer` attention over its cache and the rows of its latest
 * projection (which must have had the same n_new_cached and n_decode):
 * the step-causal mask of mdm_step_attention, output
 * out[B][n_new_cached + n_decode + R][H*d] (fp32). */
mdm_status mdm_layer_attention(mdm_ctx* ctx, int32_t layer, int32_t n_new_cached, int32_t n_decode, float* out);

/* ---- training-form attention under the block mask -----------------------
 * Page 1 (papernotes.org), key design 3; page 3 (paperlayer.ai), sections 3.3
 * and 7.3: training reproduces the incremental cache in one parallel forward.
 * Every row of a sequence carries a block id.  With M = n_clean_blocks[b]
 * (the prompt is block 0, clean tokens are blocks 1..M, masked tokens blocks
 * M+1..M+N, each masked block followed by its own copy of the registers under
 * the same id), a row of block i <= M sees the keys of blocks j <= i; a row of
 * block i > M sees its own block and every block j <= M.  Ids are labels: rows
 * may come in any order, any int32 values are allowed, and every row sees at
 * least itself.
 *
 * Inputs are the layer's RoPE'd activations (this call applies no RoPE):
 *   q       bf16 [B][n][H][head_dim]
 *   k, v    bf16 [B][n][H_kv][head_dim]
 *   blocks  int32 [B][n]
 *   n_clean_blocks  int32 [B]
 * Output: out fp32 [B][n][H][head_dim] = softmax(q k^T / sqrt(head_dim)) v
 * over the visible keys (query head h uses kv head h / (H / H_kv)).
 * q, k, v and out must be 16-byte aligned; the workspace (caller-owned,
 * mdm_block_attention_workspace_bytes, 4-byte aligned) holds per-tile block-id
 * ranges.  head_dim must be 128 and n at most 16384 (MDM_E_UNSUPPORTED);
 * MDM_E_ARG for NULL pointers, non-positive sizes, H not a multiple of H_kv or
 * misalignment; MDM_E_SHAPE for a short workspace.  No context: the call is
 * enqueued on `stream` (a hipStream_t, NULL = the default stream) and errors
 * are reported by mdm_last_error(NULL). */
typedef struct {
  int32_t batch;
  int32_t n_rows;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
} mdm_block_attn_shape;

size_t mdm_block_attention_workspace_bytes(const mdm_block_attn_shape* shape);

mdm_status mdm_block_attention(const mdm_block_attn_shape* shape, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* blocks, const int32_t* n_clean_blocks,
                               float* out, void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mdm_block_attention without a workspace argument.  The per-tile block-id
 * ranges go to a library-owned static device array of 16384 int32 (64 KiB)
 * per GPU, which each GPU holds until the process ends; the launch needs
 * 2 * batch * ceil(n_rows / 64) of them (MDM_E_UNSUPPORTED beyond, checked
 * before anything is enqueued).  The array's device address is looked up once
 * per device, on the first call with that device current.  The call allocates
 * nothing.  Every call on one GPU shares that GPU's array; each call writes
 * the ranges it reads before reading them, so nothing needs clearing, but
 * calls that overlap on one GPU (e.g. on two streams) race.  Other arguments,
 * layouts and errors as in mdm_block_attention. */
mdm_status mdm_block_attention_static(const mdm_block_attn_shape* shape, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* v, const int32_t* blocks, const int32_t* n_clean_blocks,
                                      float* out, void* stream);

/* Release the host context (device buffers stay the caller's). */
void mdm_sparse_step_destroy(mdm_ctx* ctx);

/* Message of the last error on ctx ("" if none); valid until the next call. */
const char* mdm_last_error(const mdm_ctx* ctx);

/* Static name of a status code. */
const char* mdm_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MDM_SPARSE_H */
