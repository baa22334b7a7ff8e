/*
 * orthrus.h — C ABI of the MI355X heterogeneous-batch forward step.
 *
 * One call runs one forward pass of a pre-norm decoder (RMSNorm, GQA
 * attention with rotate-half RoPE, SwiGLU FFN) over a packed, ragged batch
 * that mixes embedding chunks, generation prefill chunks and single-token
 * decode rows, then splits the outputs: next-token logits for generation,
 * incremental pooling for embedding.  This is the runner's forward + emit
 * stages as described in "Efficient Iterative Retrieval with Heterogeneous
 * Batching" (paperpeel full text), §3.1 High-Level Workflow and §3.2 Batch
 * Unit, with the pooling state of §3.3 Incremental Pooler as completed on
 * the agihunt summary page (running weighted sum + weight total, or a kept
 * hidden state).  A LoRA adapter applies to embedding rows only (§2.2
 * Parameter sharing, §5.1 Workloads, Models, and Hardware).
 *
 * Conventions
 *  - Every pointer documented "device" is device memory of the current HIP
 *    device; "host" pointers are ordinary host memory.  The caller owns all
 *    of them.  The engine owns only its workspace and pinned staging.
 *  - bf16 is IEEE bfloat16 stored as 16-bit patterns; fp32 is IEEE binary32.
 *  - Linear weights are row-major [out_features][in_features].
 *  - K and V caches are each [n_layers][n_pages][n_kv_heads][page_size]
 *    [head_dim] bf16 (fp32 for models of dtype ORTHRUS_F32).  Token
 *    position p of an item lives in page page_ids[page_off + p / page_size]
 *    at in-page offset p % page_size.
 *  - Nothing throws across this ABI.  Validation runs before any device
 *    work; on a non-OK status no device memory has been touched.
 */
#ifndef ORTHRUS_H
#define ORTHRUS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ORTHRUS_OK = 0,
  ORTHRUS_EINVAL = 1,     /* malformed batch or configuration */
  ORTHRUS_ENOPAGES = 2,   /* an item's pages cannot hold ctx_len + n_tokens, or a page id is out of range */
  ORTHRUS_ECAPACITY = 3,  /* batch exceeds max_tokens/max_items, or an output buffer is too small */
  ORTHRUS_ESTATE = 4,     /* pooling slot out of range or reused, or a first chunk not at position 0 */
  ORTHRUS_ENOMEM = 5,     /* device or pinned allocation failed */
  ORTHRUS_EHIP = 6        /* a HIP call failed; orthrus_last_error() has the HIP message */
} orthrus_status;

/* Item kinds, in the order a batch must list them (§3.2 Batch Unit: the
 * scheduler emits batches sorted by request type). */
enum { ORTHRUS_EMBED = 0, ORTHRUS_PREFILL = 1, ORTHRUS_DECODE = 2 };

/* Pooling heads (§3.3 Incremental Pooler; agihunt summary).  MEAN weights
 * every token 1; WMEAN weights a token by its 1-based position in the
 * request; CLS keeps the hidden state at position 0; LAST keeps the hidden
 * state of the request's final token.  BUFFER (the Summary page's
 * incremental-pooling paragraph: keep n x d values per request for a head
 * that is not a streaming sum) stores every final hidden state of
 * the request at its position in the slot's buffer and, on the last chunk,
 * emits the mean of all N buffered rows, summed in an order fixed by N
 * alone; the buffer stays readable for any other head.  ORTHRUS_POOL_L2,
 * OR'ed into any kind, scales the emitted vector to unit L2 length
 * (e / max(|e|, 1e-12); the OpRAG page's mean-pool-then-normalise
 * convention). */
enum { ORTHRUS_POOL_MEAN = 0, ORTHRUS_POOL_WMEAN = 1, ORTHRUS_POOL_CLS = 2, ORTHRUS_POOL_LAST = 3,
       ORTHRUS_POOL_BUFFER = 4, ORTHRUS_POOL_L2 = 8 };

typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  int32_t lora_rank;       /* 0 = no adapter; otherwise a multiple of 8 */
  int32_t page_size;       /* tokens per KV page */
  int32_t n_pages;         /* pages in each layer's K and V pool */
  int32_t max_tokens;      /* largest batch (rows) the engine accepts */
  int32_t max_items;       /* largest item count the engine accepts */
  int32_t max_pool_slots;  /* rows of the pooling state arrays */
  float rope_theta, rms_eps, lora_scale;
  int32_t dtype;           /* ORTHRUS_BF16 (0) or ORTHRUS_F32 (1), see below */
} orthrus_model_cfg;

/* Number format of a model (orthrus_model_cfg.dtype).  ORTHRUS_BF16: bf16
 * weights and KV pages, bf16 matrix-core operands with fp32 accumulation,
 * an fp32 residual stream, fp32 softmax and pooling.  ORTHRUS_F32: every
 * weight, KV page, activation and accumulation in fp32 (weight and KV
 * pointers then point to IEEE binary32 arrays of the same shapes), on
 * kernels written for correctness at small sizes (the tiny fp32 decoder),
 * not for speed. */
enum { ORTHRUS_BF16 = 0, ORTHRUS_F32 = 1 };

/* Per-layer weights, all device bf16 (fp32 when cfg.dtype is ORTHRUS_F32).
 *  w_qkv      [Hq*hd + 2*Hkv*hd][d]   q rows, then k rows, then v rows
 *  w_o        [d][Hq*hd]
 *  w_gate_up  [2*F][d]                gate rows, then up rows
 *  w_down     [d][F]
 *  g_attn, g_ffn [d]                  RMSNorm gains
 *  lora_a_qkv [3*r][d]                shrink for q, k, v (r rows each)
 *  lora_b_qkv [Hq*hd + 2*Hkv*hd][r]   expand; row n belongs to n's section
 *  lora_a_o   [r][Hq*hd], lora_b_o [d][r]
 * LoRA pointers may be NULL when lora_rank == 0. */
typedef struct {
  const void *w_qkv, *w_o, *w_gate_up, *w_down, *g_attn, *g_ffn;
  const void *lora_a_qkv, *lora_b_qkv, *lora_a_o, *lora_b_o;
} orthrus_layer_w;

/* tok_emb [V][d], lm_head [V][d], g_final [d]: device bf16 (fp32 for ORTHRUS_F32).
 * layers: host array of n_layers entries (copied by orthrus_create). */
typedef struct {
  const void *tok_emb, *lm_head, *g_final;
  const orthrus_layer_w *layers;
} orthrus_weights;

/* One batch item (host).  Rows of the batch follow item order.
 *  kind        ORTHRUS_EMBED / PREFILL / DECODE; non-decreasing over items
 *  req_id      unique within the batch
 *  n_tokens    >= 1; exactly 1 for DECODE
 *  ctx_len     tokens of this request already in the KV cache; the item's
 *              rows sit at positions ctx_len .. ctx_len + n_tokens - 1
 *  page_off, n_pages   the request's page list is page_ids[page_off ..
 *              page_off + n_pages); n_pages * page_size >= ctx_len + n_tokens
 *  pool_slot   EMBED only: row of the pooling state
 *  pool_kind   EMBED only: ORTHRUS_POOL_MEAN .. BUFFER, optionally | ORTHRUS_POOL_L2
 *  is_first    EMBED: first chunk (resets the slot; requires ctx_len == 0)
 *  is_last     EMBED: final chunk (emits the embedding); PREFILL: the chunk
 *              completes the prompt (emits logits of its last row) */
typedef struct {
  int32_t kind, req_id, n_tokens, ctx_len, page_off, n_pages;
  int32_t pool_slot, pool_kind, is_first, is_last;
} orthrus_item;

typedef struct {
  int32_t n_items, n_tokens, n_page_ids;
  const orthrus_item *items;   /* host [n_items] */
  const int32_t *token_ids;    /* host [n_tokens], item order */
  const int32_t *page_ids;     /* host [n_page_ids] */
} orthrus_batch;

/* Pooling state, device fp32: sum [max_pool_slots][d], wsum
 * [max_pool_slots], kept [max_pool_slots][d], and for the BUFFER kind
 * buf [max_pool_slots][buf_rows][d] (row p of a slot holds the final
 * hidden state of the request's token p; NULL / 0 when no BUFFER item is
 * run).  Carried across steps by the caller; a slot is private to one
 * request between its first and last chunk. */
typedef struct {
  float *sum, *wsum, *kept;
  float *buf;
  int32_t buf_rows;
} orthrus_pool_state;

/* Host metadata produced by orthrus_pack (all host int32; caller-allocated
 * with the capacities given in cap_tokens / cap_items).
 *  cu_q       [n_items+1]  row offset of each item
 *  pos        [n_tokens]   position of each row in its request
 *  slot       [n_tokens]   KV slot written by each row: page * page_size + offset
 *  row_item   [n_tokens]   item index of each row
 *  logit_rows [n_items]    rows whose logits are emitted, in item order
 *  pool_segs  [n_items*8]  per EMBED item: row_start, n_rows, pool_slot,
 *                          pool_kind, is_first, is_last, ctx_len,
 *                          output index (or -1 when not is_last) */
typedef struct {
  int32_t cap_tokens, cap_items;
  int32_t *cu_q, *pos, *slot, *row_item, *logit_rows, *pool_segs;
  int32_t n_embed_rows, n_prefill_rows, n_decode_rows, n_logits, n_emb, n_pool_segs;
} orthrus_packed;

typedef struct orthrus_engine orthrus_engine;

/* Validate a batch against cfg and build its packing metadata; host only,
 * no HIP call.  Checks run in a fixed order and the first failure is
 * returned; err (may be NULL) receives a message.  Capacity of `out`
 * arrays too small -> ORTHRUS_ECAPACITY. */
orthrus_status orthrus_pack(const orthrus_model_cfg *cfg, const orthrus_batch *batch,
                            orthrus_packed *out, char *err, int32_t err_len);

/* Create an engine bound to the current HIP device.  Copies cfg and the
 * weight pointer table; allocates the workspace for max_tokens/max_items.
 * k_pages / v_pages: device KV pools (layout above; bf16, or fp32 for
 * ORTHRUS_F32), read and written by every step.  Returns EINVAL for an
 * unknown dtype or unsupported shapes (head_dim not in
 * {16,32,64,128}, n_q_heads not a multiple of n_kv_heads, d_model above
 * 8192, d_model, Hq*hd, ffn_dim not multiples of 8, lora_rank not a
 * multiple of 8, or a step operand of 2 GiB or more: max_tokens rows of
 * the widest activation in fp32, or the vocab x d_model, 2 ffn_dim x
 * d_model or (Hq + 2 Hkv) hd x d_model weight in bf16), ENOMEM or EHIP on
 * allocation failure. */
orthrus_status orthrus_create(const orthrus_model_cfg *cfg, const orthrus_weights *w,
                              void *k_pages, void *v_pages, orthrus_engine **out);

/* Run one step on `stream` (a hipStream_t; NULL = default stream).
 * Asynchronous: outputs are valid once the stream has synchronised.  The
 * batch's host arrays may be reused as soon as the call returns.  Steps of
 * one engine run in call order: a step issued on a different stream than
 * the previous step first waits (on the device) for the previous step's
 * work, since both use the engine's workspace.  Calls on one engine from
 * several host threads at once are not supported.
 *  logits      device fp32 [logits_cap_rows][vocab]: rows in item order
 *              (prefill items with is_last, then decode items)
 *  emb         device fp32 [emb_cap_rows][d]: embedding items with is_last,
 *              in item order (the pooled vector; unit length when the
 *              item's pool kind carries ORTHRUS_POOL_L2)
 *  n_logits, n_emb   host out: rows written
 *  logit_req_ids, emb_req_ids   optional host int32 [logits_cap_rows] /
 *              [emb_cap_rows]: req_id of each logit row / embedding row,
 *              written before the call returns (NULL to skip)
 *  hidden_out  optional device fp32 [n_tokens][d]: residual stream after
 *              the last layer (NULL to skip)
 * Every row appends its K/V at its slot; pooling state is updated.
 * Errors: any orthrus_pack status; ECAPACITY when logits_cap_rows or
 * emb_cap_rows is too small or a BUFFER item reaches past pool->buf_rows
 * (or pool->buf is NULL); EHIP/ENOMEM from the runtime. */
orthrus_status orthrus_step(orthrus_engine *eng, const orthrus_batch *batch,
                            const orthrus_pool_state *pool, float *logits,
                            int32_t logits_cap_rows, float *emb, int32_t emb_cap_rows,
                            int32_t *n_logits, int32_t *n_emb, int32_t *logit_req_ids,
                            int32_t *emb_req_ids, float *hidden_out, void *stream);

/* orthrus_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, kernels and results as orthrus_step, but the step's
 * metadata and its decode-attention partial results live in a static
 * device array of 64 MiB that the library holds on every device it runs
 * on from module load to process end (its address is resolved once per
 * device by orthrus_create), and the call never calls hipMalloc, hipFree,
 * hipHostMalloc or any allocating routine.  Limits: at most 4 MiB of step
 * metadata (about 3 int32 words per row, the page ids, 8 words per item
 * and 12 per attention work entry: one per 128/(Hq/Hkv) rows of a chunk
 * per KV head, one per decode split per KV head) and 60 MiB of decode
 * partial results ((Hq/Hkv) * (2 + head_dim) * 4 bytes per decode split
 * per KV head; decode rows split their keys in pieces of 128 to 4096, the
 * largest that still gives 2048 decode workgroups);
 * beyond either, ECAPACITY before any device work, with the limit in
 * orthrus_last_error.  Every call on one device shares that device's
 * array: calls that overlap on one device (two engines on two streams,
 * or host threads) race and are not supported; calls in stream order are
 * safe, since each call writes all the scratch it reads. */
orthrus_status orthrus_step_noalloc(orthrus_engine *eng, const orthrus_batch *batch,
                                    const orthrus_pool_state *pool, float *logits, int32_t logits_cap_rows,
                                    float *emb, int32_t emb_cap_rows, int32_t *n_logits, int32_t *n_emb,
                                    int32_t *logit_req_ids, int32_t *emb_req_ids, float *hidden_out,
                                    void *stream);

/* Message of the last failed call on this engine ("" if none).  With
 * eng == NULL: the message of the last orthrus_create that failed in this
 * process ("" if none); not synchronised between threads. */
const char *orthrus_last_error(const orthrus_engine *eng);

/* Free the engine's workspace.  Waits for its pending work. */
void orthrus_destroy(orthrus_engine *eng);

/* Per-layer residual dump, for checking each layer of a deep model on its
 * own (feed a layer the GPU's own input and compare its output).  While
 * dst is set, every orthrus_step copies the fp32 residual stream after
 * layer l (rows 0 .. n_tokens-1, [n_tokens][d]) to dst + l * cap_rows * d,
 * on the step's stream.  dst: device fp32 [n_layers][cap_rows][d], owned
 * by the caller, NULL to stop.  A step with more than cap_rows rows
 * returns ECAPACITY before any device work.  EINVAL for a NULL engine or
 * cap_rows < 1 with a non-NULL dst. */
orthrus_status orthrus_set_layer_dump(orthrus_engine *eng, float *dst, int64_t cap_rows);

/* Per-kernel timing.  While enabled, every kernel launch of orthrus_step is
 * bracketed by HIP events recorded on the step's stream (the stream the
 * kernel runs on).  orthrus_profile_read waits for the recorded events,
 * writes a JSON object {"<kernel>": {"count", "total_ms", "min_ms",
 * "max_ms"}, ...} accumulated since the last read into json (truncated to
 * len-1 bytes, NUL-terminated), clears the record and returns the full
 * length, or -1 for a NULL engine.  With json NULL or len 0 it only returns
 * the length and keeps the record.  Host-side instrumentation only; the
 * kernels are unchanged. */
orthrus_status orthrus_profile(orthrus_engine *eng, int32_t enable);
int32_t orthrus_profile_read(orthrus_engine *eng, char *json, int32_t len);

/* Seeded synthetic bf16 fill (device): dst[i] = value start+i of the
 * SplitMix64 counter hash keyed by (seed, tensor_id), mapped to a uniform
 * value of unit variance and rounded to bf16:
 *   z = ((seed << 32) ^ tensor_id) + (start + i + 1) * 0x9E3779B97F4A7C15
 *   z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9; z = (z ^ (z >> 27)) * 0x94D049BB133111EB
 *   h = z ^ (z >> 31); u = (h >> 40) * 2^-24; v = bf16_rne((2u - 1) * 1.7320508f)
 * Used to lay down prior KV pages and other synthetic state of large
 * workloads without a host upload; the definition is exact, so a host
 * implementation reproduces the same bits.  Asynchronous on `stream`. */
orthrus_status orthrus_fill_hash_bf16(void *dst, uint64_t n, uint32_t seed, uint32_t tensor_id, uint64_t start,
                                      void *stream);

/* Standalone bf16 GEMM on the MFMA kernels of the step (device pointers):
 *   C = A B^T with A [M][K] (lda), B [N][K] (ldb), fp32 accumulation.
 * epilogue: 0 store C as bf16 [M][N] (ldc); 1 store fp32; 2 fp32 C += A B^T
 *             (a tile that one workgroup computes over all of K is read,
 *             added and written; where large problems split K over
 *             workgroups, the partial sums land by float atomic adds in
 *             no fixed order, so C must not be read or written by other
 *             work on the device meanwhile);
 *           3 SwiGLU: B holds 2N rows at ldb (gate rows 0..N-1, up rows
 *             N..2N-1 at row offset b_up_row), C bf16 = silu(gate) * up.
 * K must be a multiple of 8.  A, B and (epilogue 2) C are addressed
 * through 32-bit buffer offsets, so each must span less than 2 GiB.
 * Returns EINVAL for bad sizes, EHIP on launch failure.  Used by the step
 * for the projections of the forward pass (§3.1: attention and feed-forward layers are shared by all items). */
orthrus_status orthrus_gemm_bf16(const void *A, int32_t lda, const void *B, int32_t ldb,
                                 void *C, int32_t ldc, int32_t M, int32_t N, int32_t K,
                                 int32_t epilogue, int32_t b_up_row, void *stream);

/* Adapter shrink U = bf16(scale * X A^T): the first half of the low-rank
 * update that embedding rows take in the QKV and O projections (full text
 * §2.2 Parameter sharing: the embedding task shares the backbone and adds
 * a LoRA adapter; §5.1 places it on q, k, v and o).  The step runs the
 * same code; this entry point exists for tests and timing.
 *  X      device bf16 [rows][ldx], ldx >= K (the normed rows, or the
 *         attention output for the O adapter)
 *  A      device bf16 [nr][K]: the adapter's down-projection, one row per
 *         output column (nr = 3 x rank for QKV, rank for O)
 *  U      device bf16 [rows][nr] out
 *  workspace, workspace_bytes
 *         optional device scratch (NULL or too small: not used).  With
 *         at least 32 * rows * nr bytes the library may split K over up to
 *         8 workgroups per 64 x 64 tile (at most two workgroups per compute
 *         unit in all) and
 *         add their fp32 partial sums in a fixed order in a second kernel;
 *         otherwise one workgroup runs a tile's whole K with `scale` folded
 *         into the GEMM's bf16 epilogue.  Either way the result does not
 *         depend on timing.  The step uses a workspace it allocates at
 *         orthrus_create.
 * Asynchronous on `stream`; allocates nothing.  EINVAL for rows or nr < 0,
 * K < 8, K % 8, ldx < K, ldx % 8, workspace_bytes < 0, NULL pointers with
 * rows, nr > 0, or operands spanning 2 GiB or more; EHIP on launch
 * failure. */
orthrus_status orthrus_lora_shrink_bf16(const void *X, int32_t ldx, const void *A, int32_t rows,
                                        int32_t nr, int32_t K, float scale, void *U, void *workspace,
                                        int64_t workspace_bytes, void *stream);

/* Next-token choice for logit rows (full text §3.1: the emit stage hands
 * every generation request's last-row logits to the sampler; §2.2
 * Generation: one new token per decoding step).  One workgroup per row.
 *  logits       device fp32 [n_rows][ld], vocab <= ld valid columns; finite
 *  temperature  device fp32 [n_rows] or NULL (NULL: greedy for every row).
 *               A row whose temperature is not > 0 takes the greedy token:
 *               the index of its largest logit, the lowest among equal ones.
 *  top_p        device fp32 [n_rows] or NULL (= 1): nucleus share, used as
 *               P16 = rint(top_p * 65536) clamped to [1, 65536]
 *  uniforms     device uint32 [n_rows]: one uniform 32-bit draw per row;
 *               required when temperature is given
 *  tokens       device int32 [n_rows] out
 * Rows with temperature T > 0: with s = fp32(log2 e / T) and
 * t_i = (l_i - max) * s in fp32 (0 at the maximum), token i weighs
 * q_i = floor(2^(30 + t_i)) (0 below t = -30; 2^f from the fp32 Horner
 * form of the degree-7 Taylor polynomial of e^(f ln 2), no fused
 * multiply-add).  The nucleus is the smallest set of highest-weight tokens
 * (lower index first among equal weights) whose weight reaches
 * ceil(sum(q) * P16 / 65536); with its mass M and x = floor(M * U / 2^32),
 * the token is the first in index order whose running nucleus weight
 * exceeds x.  The result depends on nothing else (no summation order), so
 * it is reproducible bit for bit.  Asynchronous on `stream`; allocates
 * nothing.  EINVAL for n_rows < 0, vocab < 1, ld < vocab, NULL logits or
 * tokens (n_rows > 0), or temperature without uniforms; EHIP on launch
 * failure. */
orthrus_status orthrus_sample(const float *logits, int64_t ld, int32_t n_rows, int32_t vocab,
                              const float *temperature, const float *top_p, const uint32_t *uniforms,
                              int32_t *tokens, void *stream);

/* ---- Intra-batch scheduler and host step driver (host only) -------------
 * Full text §4 Intra-Batch Scheduling.  Each call of orthrus_sched_next
 * builds the next batch: one row for every generation request in its decode
 * phase (submission order; a decode that needs a KV page when none is free
 * waits), then the residual token budget filled from the embedding queue and
 * the generation (prompt) queue.  The queue is chosen by credit
 * accumulators: a_e += w_e, a_g += w_g with w_e, w_g the queues' unscheduled
 * input tokens at the start of the fill; the larger credit wins (ties to
 * embedding) and loses w_e + w_g; a queue empty at the start of a step has
 * its credit reset.  The chosen queue offers its next request not yet
 * scheduled in this step, as a chunk of min(C, unscheduled tokens); if that
 * does not fit the budget, the free pages or (first embedding chunk) the
 * free pooling slots, the queue closes for the step (strict FCFS) and the
 * selection's credit change is undone.  The batch lists embedding chunks,
 * prompt chunks, then decode rows, each in submission order; its page lists
 * come from the scheduler's FIFO free list (pages return to its back when a
 * request finishes; pooling slots likewise).  A generation request with
 * max_new_tokens m takes its first token from the logits of the chunk that
 * completes its prompt and then runs m - 1 decode rows. */
typedef struct orthrus_sched orthrus_sched;

/* token_budget B >= 1 rows per step, chunk C >= 1, page_size >= 1;
 * free_pages: host [n_free_pages], the initial free-list order (copied);
 * pooling slots 0 .. n_pool_slots-1.  EINVAL on bad arguments. */
orthrus_status orthrus_sched_create(int32_t token_budget, int32_t chunk, int32_t page_size,
                                    const int32_t *free_pages, int32_t n_free_pages,
                                    int32_t n_pool_slots, orthrus_sched **out);

/* Queue a request (tokens copied).  kind ORTHRUS_EMBED (pool_kind one of
 * ORTHRUS_POOL_*) or ORTHRUS_PREFILL (a generation request, max_new_tokens
 * >= 1).  EINVAL for a bad kind, pool kind, length or token count, or a
 * req_id submitted before. */
orthrus_status orthrus_sched_submit(orthrus_sched *s, int32_t req_id, int32_t kind,
                                    const int32_t *tokens, int32_t n_tokens, int32_t pool_kind,
                                    int32_t max_new_tokens);

/* Build the next batch into *out (n_items == 0 when nothing can run).  The
 * arrays *out points to are owned by the scheduler and stay valid until the
 * next orthrus_sched_commit.  *n_logits: logit rows of the batch.  ESTATE
 * while the previous batch has not been committed. */
orthrus_status orthrus_sched_next(orthrus_sched *s, orthrus_batch *out, int32_t *n_logits);

/* Advance after the batch ran: sampled[k] is the token chosen from logit
 * row k (the batch's logit rows in item order).  EINVAL unless n_sampled
 * equals the batch's logit rows; ESTATE without a pending batch. */
orthrus_status orthrus_sched_commit(orthrus_sched *s, const int32_t *sampled, int32_t n_sampled);

/* out8: embedding requests queued, prompt requests queued, requests
 * decoding, free pages, free pooling slots, credit a_e, credit a_g,
 * batch pending (0/1). */
orthrus_status orthrus_sched_stats(const orthrus_sched *s, int64_t *out8);

void orthrus_sched_destroy(orthrus_sched *s);

#ifdef __cplusplus
}
#endif

#endif /* ORTHRUS_H */
