/*
 * pkv.h — C ABI of the MI355X (gfx950) paged-KV GQA decode path.
 *
 * The library computes the batched decode step of a Llama/Qwen-style
 * grouped-query-attention decoder over one shared BF16 KV page pool, as the
 * "Inference from Scratch" engine summary describes it (page "Hours of
 * YouTube and 85 handtyped pages of notes on LLM Inference", its feature
 * bullets on the page pool, paged attention, batched decode and the final
 * norm): pages of 16 tokens of BF16 K and V, one block table per sequence
 * and layer; each decode step writes the new token's K and V at its
 * absolute RoPE position; attention reads the cached pages in place through
 * the block table, keeping the softmax running in FP32, so neither a copied
 * contiguous cache nor a score matrix ever exists; every active sequence
 * contributes one token to a step; a final RMSNorm and the tied embedding
 * matrix give FP32 logits, whose argmax is taken on the GPU.  The
 * configuration fields are those of llmc's binary header (README of llmc,
 * section "binary format v2", config header).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  BF16 data are
 *     passed as uint16_t bit patterns.  All arrays are dense row-major.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; no call synchronises except pkv_device_error.
 *   - The caller owns every buffer (pool, weights, tables, activations,
 *     logits, workspace).  The library allocates and frees nothing and keeps
 *     no pointer after a call returns.  Buffers must stay alive until the
 *     stream has passed the enqueued work.
 *   - Errors are negative errno values, as in llmc's kernel-style convention
 *     (README of llmc: every operator returns a negative errno on error):
 *       0        success
 *       -EINVAL  NULL pointer, bad shape, inconsistent sizes, misalignment
 *       -ENOTSUP head_dim not 64 or 128, page_tokens not 16 or 256, or a size outside what
 *                this version supports (stated per call)
 *       -ENOSPC  pool smaller than one page, workspace too small
 *       -EIO     the HIP runtime rejected a launch (the error is cleared)
 *     Argument validation is host code that runs before any HIP call.
 *   - Errors that only the device can see (a block-table entry outside
 *     [0, num_pages), a position or length beyond the table or the RoPE
 *     table, a token id outside the vocabulary) set bits of a sticky word in
 *     the workspace (PKV_DEVERR_*); the offending page, token or sequence is
 *     skipped and the corresponding outputs are unspecified.  Read and clear
 *     the word with pkv_device_error.
 *   - A workspace must be zero-initialised once (pkv_workspace_init) before
 *     its first use; the kernels leave it ready for the next call, of any
 *     entry point and any shape that fits it.  Its first 2304 bytes are a
 *     header that every call's layout leaves to the error word and to the
 *     single-launch layer's launch counters (decoder_layer_decode), whose
 *     exchange words carry tagged launch numbers that no other stored value
 *     has.  Calls that share a workspace must be ordered on one stream;
 *     calls on different streams need different workspaces.
 *
 * Pool layout: a page of PT tokens (page_tokens: 16, the engine's page, or
 * 256, the fixed page length of the three-stage engine's paged KV cache)
 * holds, as BF16, a K block and a V block, both in 16-token tiles so that a
 * tile of one kv head is one contiguous matrix-core operand at any page
 * size:
 *   K [PT / 16][num_kv_heads][head_dim / 8][16 slots][8 dims]: each token's
 *     dimensions in chunks of 8, the 16 slots' chunk c side by side (the
 *     score product's operand, read 1 KiB per load instruction);
 *   V [PT / 16][num_kv_heads][head_dim][16 slots]: V transposed within a
 *     tile (the value product's operand).
 * With one buffer (kv_pool_create) physical page p starts at
 * base + p * page_bytes with its K block followed by its V block, page_bytes =
 * 2 * num_kv_heads * PT * head_dim * 2 (32 KiB for 16 tokens of 8 kv heads
 * of width 64, 64 KiB at width 128, 8 KiB for 2 heads of width 64).  With
 * separate K and V pools (kv_pool_create_split, as the three-stage engine
 * keeps its K and V caches apart) page p's K block is at
 * base + p * page_bytes and its V block at v_base + p * page_bytes,
 * page_bytes = num_kv_heads * PT * head_dim * 2.
 * Token t of a sequence lives in logical page t / PT, slot t % PT; the
 * sequence's block-table row maps the logical page to a physical page.
 * Block tables are int32 [batch][max_pages] per layer; decode_step takes
 * them layer-major, [num_layers][batch][max_pages].  Entries past a
 * sequence's last page are never read.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_PAGE_TOKENS 16
#define PKV_HEAD_DIM 64     /* the default head width; 128 is also supported */

/* Packed weight layouts (pkv_pack_weight). */
#define PKV_PACK_ROWS 0     /* rows in order: w_o, w_down, embed / LM head   */
#define PKV_PACK_QKV 1      /* w_qkv: the RoPE pairs of a head grouped        */
#define PKV_PACK_GATE_UP 2  /* w_gate_up: 8 gate rows with their 8 up rows    */
#define PKV_PACK_QKV128 3   /* w_qkv of 128-wide heads, pairs grouped alike   */

/* Sticky device-error bits (pkv_device_error). */
#define PKV_DEVERR_PAGE 1u      /* block-table entry outside [0, num_pages) */
#define PKV_DEVERR_LENGTH 2u    /* length / position beyond max_pages * PT  */
#define PKV_DEVERR_ROPE 4u      /* position >= max_position_embeddings      */
#define PKV_DEVERR_TOKEN 8u     /* token id outside [0, vocab_size)         */
#define PKV_DEVERR_SYNC 16u     /* single-launch layer: a phase's input did not
                                   arrive in time (outputs unspecified)      */

/* Model configuration: the config-header fields of llmc's binary format. */
typedef struct pkv_config {
	int32_t hidden_size;             /* H, multiple of 64                  */
	int32_t num_hidden_layers;       /* layers (decode_step)              */
	int32_t num_attention_heads;     /* Hq                                 */
	int32_t num_key_value_heads;     /* Hkv, divides Hq                    */
	int32_t head_dim;                /* D, 64 or 128                       */
	int32_t intermediate_size;       /* I, multiple of 64                  */
	int32_t vocab_size;              /* V (decode_step)                    */
	int32_t max_position_embeddings; /* rows of the RoPE cos/sin tables    */
	float rope_theta;                /* RoPE base                          */
	float rms_norm_eps;              /* RMSNorm epsilon (inside the root)  */
} pkv_config;

/* A view of caller-allocated device buffers as a page pool (no ownership). */
typedef struct pkv_pool {
	void *base;           /* device, 256-byte aligned                         */
	int64_t bytes;        /* size of the buffer                               */
	int64_t page_bytes;   /* per page and buffer: K + V, or one of them      */
	int32_t num_pages;    /* floor(bytes / page_bytes)                        */
	int32_t page_tokens;  /* 16 or 256                                        */
	int32_t num_kv_heads; /* Hkv                                              */
	int32_t head_dim;     /* 64 or 128                                        */
	void *v_base;         /* NULL: K and V in one buffer; else the V pool     */
} pkv_pool;

/*
 * One layer's weights, BF16, no biases.  The norms are plain [H] vectors;
 * the four matrices are given by their row-major [out][in] form (the
 * Hugging Face orientation) and passed PACKED (pkv_pack_weight, once, at
 * load time):
 *   attn_norm [H], mlp_norm [H]                  RMSNorm weights
 *   w_qkv     [(Hq + 2 Hkv) * D][H]              q rows, then k rows, then v rows;
 *                                                packed PKV_PACK_QKV (D = 64)
 *                                                or PKV_PACK_QKV128 (D = 128)
 *   w_o       [H][Hq * D]                        packed PKV_PACK_ROWS
 *   w_gate_up [2 I][H]                           gate rows, then up rows;
 *                                                packed PKV_PACK_GATE_UP
 *   w_down    [H][I]                             packed PKV_PACK_ROWS
 */
typedef struct pkv_layer_weights {
	const uint16_t *attn_norm, *w_qkv, *w_o, *mlp_norm, *w_gate_up, *w_down;
} pkv_layer_weights;

/*
 * Whole-model weights.  embed [V][H] BF16, packed PKV_PACK_ROWS, is both
 * the embedding table (rows gathered by token id) and the LM head (tied).
 * layers is a HOST array of num_hidden_layers entries.  rope_cos/rope_sin
 * are device FP32 tables [max_position_embeddings][D/2] (pkv_rope_table).
 */
typedef struct pkv_model_weights {
	const uint16_t *embed, *final_norm;
	const pkv_layer_weights *layers;
	const float *rope_cos, *rope_sin;
} pkv_model_weights;

/*
 * kv_pool_create — describe a caller-owned device buffer as a page pool
 * (the engine's shared BF16 page pool sized in bytes, its --kv-cache-mib
 * option).  No device work, no allocation; `out` is a host struct.
 * Errors: -EINVAL (NULL, misaligned base, bytes < 0, num_kv_heads < 1),
 * -ENOTSUP (head_dim not 64 or 128, or page_tokens not 16 or 256), -ENOSPC
 * (less than one page, or more than INT32_MAX pages).
 */
int kv_pool_create(void *dev_base, int64_t bytes, int32_t num_kv_heads,
		   int32_t head_dim, int32_t page_tokens, pkv_pool *out);

/*
 * kv_pool_create_split — the same over two caller-owned device buffers of
 * `bytes` bytes each, K blocks in k_base and V blocks in v_base, both
 * 256-byte aligned and not overlapping (the three-stage engine's paged KV
 * cache keeps separate K and V caches indexed by one page number, its
 * section 3.2).  Every call that takes a pool accepts either kind.
 * Errors: as kv_pool_create; -EINVAL also for v_base NULL or overlapping.
 */
int kv_pool_create_split(void *k_base, void *v_base, int64_t bytes,
			 int32_t num_kv_heads, int32_t head_dim,
			 int32_t page_tokens, pkv_pool *out);

/*
 * kv_append — write one new token's K and V per sequence into the pool at
 * its absolute position (decode appends one token at its RoPE position).
 *   block_table [batch][max_pages] int32, positions [batch] int32,
 *   k_new, v_new [batch][Hkv][D] BF16.
 * Sequence b writes slot positions[b] % PT of physical page
 * block_table[b][positions[b] / PT].  Bit-exact copy of the given values.
 * A sequence whose position is negative or past the table
 * (PKV_DEVERR_LENGTH) or whose table entry lies outside [0, num_pages)
 * (PKV_DEVERR_PAGE) writes nothing; the bit is ORed into *dev_error, a
 * device word the caller owns (for instance the first word of a workspace,
 * read and cleared with pkv_device_error), or dropped if dev_error is NULL.
 * batch == 0 is a no-op.  Errors: -EINVAL, -ENOTSUP, -EIO.
 */
int kv_append(const pkv_pool *pool, const int32_t *block_table,
	      int32_t max_pages, const int32_t *positions,
	      const uint16_t *k_new, const uint16_t *v_new, int32_t batch,
	      uint32_t *dev_error, void *stream);

/*
 * paged_gqa_decode — decode attention read straight from the pages, with an
 * FP32 online softmax ("Inference from Scratch" summary, paged-attention
 * bullet: the kernel walks a sequence's block table and folds every cached
 * token into a running maximum, normaliser and weighted sum of V, so the
 * pages are never copied into one buffer and no score is written out).
 *   q [batch][num_q_heads][D] BF16, context_lens [batch] int32 (tokens
 *   0..n-1 are attended), out [batch][num_q_heads][D] FP32.
 * Query head h reads kv head h / (num_q_heads / Hkv).  For every head:
 *   out = sum_t softmax_t(scale * q.K_t) V_t  over t < n.
 * n == 0 gives zeros.  The result does not depend on where the pages lie
 * in the pool, on the page size or on the pool kind (work is split on
 * 16-token tiles of the logical sequence).  D is the pool's head width.
 * workspace: at least pkv_attention_workspace_bytes(...) bytes for the
 * pool's head width and page size, initialised once.
 * Errors: -EINVAL (NULL, Hq % Hkv != 0, batch < 0, max_pages < 1),
 * -ENOTSUP (Hq / Hkv > 16, batch > 65535, max_pages * PT > 8388480), -ENOSPC
 * (workspace), -EIO; device errors PKV_DEVERR_PAGE, PKV_DEVERR_LENGTH.
 */
int paged_gqa_decode(const pkv_pool *pool, const uint16_t *q,
		     int32_t num_q_heads, const int32_t *block_table,
		     int32_t max_pages, const int32_t *context_lens,
		     int32_t batch, float scale, float *out, void *workspace,
		     size_t ws_bytes, void *stream);

/*
 * paged_gqa_decode_noalloc — paged_gqa_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * paged_gqa_decode, without the workspace: the split records live in a
 * fixed device array of PKV_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends, and the device-error bits
 * (PKV_DEVERR_PAGE, PKV_DEVERR_LENGTH) are ORed into *dev_error, a 4-byte
 * device word the caller owns and clears.  The call allocates nothing and
 * frees nothing.  All calls on one GPU share its array: calls that overlap
 * on one GPU (other streams, other threads) race and must not be issued.
 * Errors: as paged_gqa_decode, with -EINVAL for a NULL or misaligned
 * dev_error and -ENOSPC when the call's split records would exceed the array
 * (batch * Hkv * splits * (32 + 16 * D) * 4 bytes, splits = the table's
 * 16-token tiles / 8, or / 16 from 4096 workgroups; e.g. 16 sequences of 8
 * kv heads of width 64 over 2048-token tables take 8.65 MB); -EIO if the
 * array's device address cannot be found.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
int paged_gqa_decode_noalloc(const pkv_pool *pool, const uint16_t *q,
			     int32_t num_q_heads, const int32_t *block_table,
			     int32_t max_pages, const int32_t *context_lens,
			     int32_t batch, float scale, float *out,
			     uint32_t *dev_error, void *stream);

/*
 * decoder_layer_decode — one decoder layer for a batch of sequences, each
 * with one new token at positions[b] (tokens 0..positions[b]-1 already in
 * the pool).  In order (the engine's layer op list):
 *   xn = RMSNorm(x) * attn_norm;  [q;k;v] = W_qkv xn;  RoPE on q and k at
 *   positions[b] (pairs (j, j + D/2), angle positions[b] * theta^(-2j/D),
 *   cos/sin read from the tables);  append BF16(k), BF16(v) at
 *   positions[b];  o = attention over 0..positions[b];  h1 = x + W_o o;
 *   hn = RMSNorm(h1) * mlp_norm;  a = silu(gate) * up with [gate; up] =
 *   W_gate_up hn;  x <- h1 + W_down a.
 *   hidden [batch][H] FP32, in/out.  block_table: this layer's
 *   [batch][max_pages].  rope_cos/rope_sin [max_position_embeddings][D/2].
 * Contractions accumulate in FP32 with FP32 activations (split into two
 * BF16 halves for the matrix cores).  Errors: as paged_gqa_decode plus
 * -EINVAL (the pool's kv heads or head width differ from the config's),
 * -ENOTSUP (H or I not a multiple of 64 or above 65536, a weight matrix
 * above 2 GiB); device errors PKV_DEVERR_PAGE, PKV_DEVERR_LENGTH,
 * PKV_DEVERR_ROPE.  workspace: at least pkv_workspace_bytes(cfg, batch,
 * max_pages, pool page size) bytes, initialised once.
 * At batch 1 the layer runs as ONE launch when it fits (pkv_fused_layer_plan;
 * the engine-building article, section 4.2, on the cost of a layer's many
 * small launches): one workgroup per compute unit, every workgroup resident
 * at once, the layer's weights streamed into LDS at kernel start and the
 * phases passing their small vectors through the workspace; nothing else may
 * occupy the GPU's compute units meanwhile, or a phase can wait past its
 * bounded deadline (PKV_DEVERR_SYNC, outputs unspecified).  Its products are
 * the multi-launch path's (matrix-core products of the BF16 weights with the
 * activations as BF16 hi and lo halves) summed in another order, so the two
 * agree to rounding, not bit for bit.
 */
int decoder_layer_decode(const pkv_config *cfg, const pkv_layer_weights *w,
			 const float *rope_cos, const float *rope_sin,
			 const pkv_pool *pool, const int32_t *block_table,
			 int32_t max_pages, const int32_t *positions,
			 int32_t batch, float *hidden, void *workspace,
			 size_t ws_bytes, void *stream);

/*
 * decode_step — the whole batched decode step: x = embed[token_ids[b]]
 * (BF16 widened to FP32), every layer as decoder_layer_decode with
 * block_tables[l], then the final RMSNorm, the tied LM head
 * logits = embed . xn in FP32, and next_tokens[b] = argmax (lowest index
 * among equal maxima).
 *   block_tables [num_layers][batch][max_pages], positions [batch],
 *   token_ids [batch], logits [batch][V] FP32 or NULL (not written),
 *   next_tokens [batch] int32.
 * Errors: as decoder_layer_decode; device error PKV_DEVERR_TOKEN too.
 */
int decode_step(const pkv_config *cfg, const pkv_model_weights *w,
		const pkv_pool *pool, const int32_t *block_tables,
		int32_t max_pages, const int32_t *positions,
		const int32_t *token_ids, int32_t batch, float *logits,
		int32_t *next_tokens, void *workspace, size_t ws_bytes,
		void *stream);

/*
 * prefill — dense causal prefill of one sequence's prompt into the pool
 * ("Inference from Scratch": prefill fills the prompt's pages, attention is
 * causal; one prompt at a time).  token_ids[t] is at position
 * start_pos + t; positions 0 .. start_pos-1 must already be in the pool.
 * Every layer projects all num_tokens tokens together (tiled matrix-core
 * GEMMs over the prompt), appends their BF16 K and V to the sequence's
 * pages exactly where kv_append would put them, and lets token t attend to
 * positions 0 .. start_pos + t.  Afterwards the final RMSNorm and the tied
 * LM head give the last token's FP32 logits and next_token[0] = their
 * argmax.  The result is that of num_tokens successive decode steps of this
 * sequence up to FP32 summation order (activations keep ~16 significant
 * bits, as in decode_step).
 *   block_tables [num_layers][max_pages]: this sequence's table per layer,
 *   mapping every page up to position start_pos + num_tokens - 1.
 *   token_ids [num_tokens] (device), logits [vocab_size] FP32 or NULL,
 *   next_token [1] int32.  workspace: at least
 *   pkv_prefill_workspace_bytes(cfg, num_tokens, max_pages) bytes.
 * The RoPE tables must cover start_pos + num_tokens positions.
 * num_tokens == 0 is a no-op.  Errors: -EINVAL (NULL, negative sizes,
 * start_pos + num_tokens past the table or max_position_embeddings),
 * -ENOTSUP (num_tokens > 65535, a prompt whose packed activations exceed
 * 2 GiB, unsupported sizes as decoder_layer_decode), -ENOSPC (workspace),
 * -EIO; device errors PKV_DEVERR_PAGE, PKV_DEVERR_LENGTH, PKV_DEVERR_ROPE and
 * PKV_DEVERR_TOKEN as decode_step.
 */
int prefill(const pkv_config *cfg, const pkv_model_weights *w,
	    const pkv_pool *pool, const int32_t *block_tables,
	    int32_t max_pages, int32_t start_pos, const int32_t *token_ids,
	    int32_t num_tokens, float *logits, int32_t *next_token,
	    void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes prefill needs (0 for an invalid config or size). */
size_t pkv_prefill_workspace_bytes(const pkv_config *cfg, int32_t num_tokens,
				   int32_t max_pages);

/*
 * sample_tokens — draw each sequence's next token from its logits, the
 * decoding step after the LM head ("手写LLM推理引擎" §3.3 logits
 * post-processing: temperature, softmax, top-p, a multinomial draw; §2.4:
 * top-p keeps the smallest set of tokens whose cumulative probability
 * reaches p; llmc 五: temperature / top-k / top-p after greedy).  For
 * sequence b:
 *   z = logits[b] / temperature[b]; p = softmax(z);
 *   nucleus = the smallest prefix of the tokens by decreasing p (equal
 *   logits: lower index first) whose cumulative p reaches top_p[b] (at least
 *   one token; top_p >= 1 keeps all), then at most top_k[b] of them
 *   (top_k <= 0: no limit);
 *   tokens[b] = the first nucleus token, in vocabulary order, whose
 *   cumulative p renormalised over the nucleus exceeds u[b] in [0, 1).
 * temperature[b] <= 0 is greedy (the first maximum).  u is the caller's
 * uniform draw, so the random stream is the caller's; the result is a
 * deterministic function of the inputs (probabilities are summed in 64-bit
 * fixed point, 2^-32 of the largest one).
 *   logits [batch][vocab] FP32 (device; finite values or -inf, at least one
 *   finite per row), temperature, top_p, u [batch] FP32, top_k [batch]
 *   int32, tokens [batch] int32 (device).  workspace: at least
 *   pkv_sample_workspace_bytes(batch, vocab) bytes, 256-byte aligned (about
 *   8 bytes per logit, room for every token as a candidate of the final
 *   selection, plus 24 KiB per sequence).
 * batch == 0 is a no-op.  Errors: -EINVAL (NULL, misaligned workspace,
 * vocab < 1, batch < 0), -ENOTSUP (batch > 65535), -ENOSPC, -EIO.
 */
int sample_tokens(const float *logits, int32_t batch, int32_t vocab,
		  const float *temperature, const float *top_p,
		  const int32_t *top_k, const float *u, int32_t *tokens,
		  void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes sample_tokens needs (0 for bad sizes). */
size_t pkv_sample_workspace_bytes(int32_t batch, int32_t vocab);

/*
 * Packed weight layout (used by every matrix the projections stream): the
 * matrix is cut into groups of 16 rows and its columns into 32-wide steps;
 * block (group G, step s) is 1 KiB, and its 16-byte chunk l = 16 i + m
 * holds the 8 values W[row(G, m)][32 s + 8 i .. 32 s + 8 i + 7].  Blocks
 * are ordered group-major, step-minor, so a group's columns are
 * contiguous.  row(G, m) by layout (rows past the matrix are zero):
 *   PKV_PACK_ROWS     16 G + m
 *   PKV_PACK_QKV      head G / 4, j = 8 (G % 4) + (m % 8): row 64 head + j
 *                     for m < 8, row 64 head + 32 + j for m >= 8 (the RoPE
 *                     pairs of a head sit in one group)
 *   PKV_PACK_QKV128   the same for 128-wide heads: head G / 8,
 *                     j = 8 (G % 8) + (m % 8), rows 128 head + j and
 *                     128 head + 64 + j
 *   PKV_PACK_GATE_UP  i = 8 G + (m % 8): gate row i for m < 8, up row I + i
 *                     for m >= 8 (I = rows / 2)
 * Each projection then reads whole 1 KiB blocks in the matrix-core operand
 * order, which keeps every load instruction inside one 4 KiB page.
 */

/*
 * Bytes of a packed [rows][cols] matrix (0 if cols is not a positive
 * multiple of 32, rows < 1, or rows does not suit the layout: a multiple of
 * 64 for PKV_PACK_QKV, of 128 for PKV_PACK_QKV128, of 16 for
 * PKV_PACK_GATE_UP).
 */
size_t pkv_packed_weight_bytes(int32_t rows, int32_t cols, int32_t layout);

/*
 * pkv_pack_weight — write the packed form of a row-major BF16 matrix src
 * [rows][cols] into dst (device, pkv_packed_weight_bytes bytes, 16-byte
 * aligned; src and dst must not overlap).  Errors: -EINVAL (NULL,
 * misaligned, bad sizes or layout), -ENOTSUP (matrix over 2 GiB), -EIO.
 */
int pkv_pack_weight(const uint16_t *src, int32_t rows, int32_t cols,
		    int32_t layout, uint16_t *dst, void *stream);

/*
 * Workspace bytes decoder_layer_decode / decode_step need for block tables
 * of max_pages pages of page_tokens (16 or 256) tokens (0 on bad args).
 */
size_t pkv_workspace_bytes(const pkv_config *cfg, int32_t batch,
			   int32_t max_pages, int32_t page_tokens);

/* Workspace bytes paged_gqa_decode needs, likewise (0 on bad args). */
size_t pkv_attention_workspace_bytes(int32_t num_q_heads, int32_t num_kv_heads,
				     int32_t head_dim, int32_t batch,
				     int32_t max_pages, int32_t page_tokens);

/* Zero a workspace with a fill kernel (no memset node; graph-safe). */
int pkv_workspace_init(void *workspace, size_t ws_bytes, void *stream);

/*
 * pkv_rope_table — fill cos/sin [max_pos][D/2] FP32 on the device with
 * cos(p * theta^(-2j/D)) and sin(...) evaluated in double and rounded to
 * FP32 (the article's RoPE section precomputes such tables once; here in
 * FP32 rather than FP16).  Errors: -EINVAL, -ENOTSUP (D not 64 or 128),
 * -EIO.
 */
int pkv_rope_table(float theta, int32_t head_dim, int32_t max_pos,
		   float *cos_out, float *sin_out, void *stream);

/*
 * pkv_device_error — synchronise `stream`, return the sticky device-error
 * bits (>= 0) of the workspace and clear them; -EINVAL / -EIO on failure.
 */
int pkv_device_error(void *workspace, void *stream);

/*
 * Measurement helpers: kernels that do none of the method's arithmetic, so
 * that the path's kernels can be read against what the memory system and
 * the launch path give on the same GPU.  None of them writes memory (sink
 * is a device float the kernels never store to in practice; it only keeps
 * the loads alive).
 *   pkv_probe_read        one launch that streams `bytes` bytes at buf
 *                         (16-byte aligned, a multiple of 16) once with
 *                         16-byte non-temporal loads over `workgroups`
 *                         workgroups of 256 threads: the practical read
 *                         ceiling of a launch of that size.
 *   pkv_probe_paged_read  one launch with paged_gqa_decode's grid that
 *                         issues exactly that call's K and V loads for the
 *                         same pool, table and lengths, and no arithmetic:
 *                         the ceiling of the call's data phase.
 *   pkv_probe_empty       `launches` empty kernels of `workgroups` one-wave
 *                         workgroups: the cost of a launch.
 * Errors: -EINVAL for NULL, misaligned or out-of-range arguments (the paged
 * probe validates as paged_gqa_decode), -EIO.
 */
int pkv_probe_read(const void *buf, int64_t bytes, int32_t workgroups,
		   float *sink, void *stream);
int pkv_probe_paged_read(const pkv_pool *pool, int32_t num_q_heads,
			 const int32_t *block_table, int32_t max_pages,
			 const int32_t *context_lens, int32_t batch,
			 float *sink, void *stream);
int pkv_probe_empty(int32_t launches, int32_t workgroups, void *stream);

/*
 * pkv_set_fused_layer — switch the single-launch batch-1 layer on (enable
 * != 0, the default) or off for every later call in the process; returns
 * the previous setting (1 or 0).  Off, batch-1 layers take the multi-launch
 * path (six or seven kernels per layer).  Host only, no device work.
 */
int pkv_set_fused_layer(int32_t enable);

/*
 * pkv_fused_layer_plan — 1 if decoder_layer_decode / decode_step calls with
 * this configuration, batch and block-table size run each layer as one
 * launch on a GPU of `compute_units` compute units (batch 1, hidden size at
 * most 2048, each worker wave's share of its workgroup's weights fits its
 * 33 KiB of LDS slots with one workgroup per compute unit, at most one
 * 128-token attention unit per workgroup, the phase vectors fit the
 * kernel's 22 KiB staging buffer), 0 if they take the multi-launch
 * path; -EINVAL / -ENOTSUP on bad arguments.  Host only.  The Qwen2.5-0.5B
 * shape fits at 128-token tables on 256 compute units; the Llama-3.2-1B
 * shape does not (123 MB of layer weights).
 */
int pkv_fused_layer_plan(const pkv_config *cfg, int32_t batch,
			 int32_t max_pages, int32_t page_tokens,
			 int32_t compute_units);

/* Library version string (host). */
const char *pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
