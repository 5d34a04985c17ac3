/*
 * ubd.h - C ABI of libubd, a gfx950 (MI355X) implementation of one
 * llama_decode step of a Llama-architecture transformer over ubatches with
 * a KV cache.
 *
 * The calls follow the problem statement of the pages this library is built
 * from:
 *   [ENG]  "llama.cpp AI LLM Engine - how it works" (romankryvolapov.pages.dev)
 *   [ARCH] "llama.cpp Architecture" (codeloopback.dev)
 *   [DEC]  "Decode loop: batching, KV cache, memory management" (readoss.com)
 *
 * General rules
 *   - Every call is host-side and single-threaded per context.  GPU work is
 *     enqueued on the stream given at creation (NULL = the null stream) and
 *     may still be running when a call returns; every reader of results
 *     (logits, greedy ids, KV reads) synchronises that stream first.
 *   - Pointers named "host" are host memory; "device" pointers are HIP
 *     device memory of the model's device.  The library never frees memory
 *     the caller passed in.
 *   - No call aborts the process on user error.  Constructors return NULL
 *     and set *status; other calls return the codes documented below.
 *     ubd_last_error() gives a message for the most recent failure on the
 *     calling thread.
 */
#ifndef UBD_H
#define UBD_H

#include <stdbool.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ubd_token;
typedef int32_t ubd_pos;
typedef int32_t ubd_seq_id;

/* Storage types.  q8_0 is the 32-value int8 block with one f16 scale per
 * block ([ARCH] Example 2: 34 bytes per 32 values); value = scale * code. */
typedef enum ubd_type {
    UBD_TYPE_F32 = 0,
    UBD_TYPE_F16 = 1,
    UBD_TYPE_BF16 = 2,
    UBD_TYPE_Q8_0 = 3,
} ubd_type;

/* Largest n_seq_max accepted ([ENG] Step 7: n_seq_max must fit the
 * library's sequence limit). */
#define UBD_MAX_SEQ 256

/* decode return codes ([ENG] Steps 11-12; [DEC] "Error recovery and state
 * rollback") */
#define UBD_OK 0
#define UBD_NO_KV_SLOT 1     /* no room in the KV cache; state unchanged   */
#define UBD_ABORTED 2        /* abort callback; done ubatches are kept     */
#define UBD_INVALID -1       /* invalid batch or argument; state unchanged */
#define UBD_ALLOC_FAILED -2  /* allocation / internal failure              */
#define UBD_COMPUTE_FAILED -3 /* kernel or HIP failure; ubatch rolled back */

/* ------------------------------------------------------------------ model */

/* Hyperparameters ([ENG] Step 4 key list; [ARCH] Example 8 print_info).
 * Derived: head_dim = n_embd / n_head, n_gqa = n_head / n_head_kv. */
typedef struct ubd_hparams {
    int32_t n_layer;
    int32_t n_embd;
    int32_t n_head;
    int32_t n_head_kv;
    int32_t n_ff;
    int32_t n_vocab;
    int32_t n_ctx_train;
    float rms_eps;          /* RMSNorm epsilon (inside the square root)    */
    float rope_freq_base;   /* RoPE theta base                             */
    int32_t rope_type;      /* 0 = normal (adjacent pairs); only 0 exists  */
} ubd_hparams;

/* One weight tensor, named as in GGUF ([ENG] Step 6):
 *   token_embd.weight, output_norm.weight, output.weight and, for every
 *   layer N, blk.N.{attn_norm, attn_q, attn_k, attn_v, attn_output,
 *   ffn_norm, ffn_gate, ffn_up, ffn_down}.weight
 * Shapes use ggml's order ([ARCH] Example 4): ne[0] = values per row (the
 * input dimension), ne[1] = rows (the output dimension); norm gains have
 * ne = {n_embd, 1}.  Norm gains must be F32.  All 2-D matrices of a model
 * share one storage type: F32 (F16 sources are widened to it exactly), BF16
 * or Q8_0.
 *   F32 / F16 / BF16: data = ne[1] rows of ne[0] values, row-major.
 *   Q8_0: data = int8 codes [ne[1]][ne[0]] and scales = f16 bit patterns
 *         [ne[1]][ne[0] / 32]; or scales = NULL and data = the GGUF block
 *         layout, [ne[1]][ne[0] / 32] blocks of 34 bytes (f16 scale, then
 *         32 codes).  ne[0] must be a multiple of 32.
 * output.weight may be left out: the model is then tied and its logits
 * use token_embd.weight as the output matrix ([ENG] Step 6: the output
 * tensor is optional and duplicates the embedding when absent).
 * data / scales are host pointers unless on_device != 0.  They are copied
 * during ubd_model_load and may be freed afterwards. */
typedef struct ubd_tensor_src {
    const char *name;
    ubd_type type;
    int64_t ne[2];
    const void *data;
    const void *scales;
    int32_t on_device;
} ubd_tensor_src;

/* Device allocation hooks: alloc returns device memory of >= nbytes
 * (256-byte aligned) or NULL; free releases it.  NULL hooks = hipMalloc /
 * hipFree. */
typedef void *(*ubd_alloc_fn)(size_t nbytes, void *user_data);
typedef void (*ubd_free_fn)(void *ptr, void *user_data);

typedef struct ubd_model_params {
    int32_t device;         /* HIP device ordinal                          */
    ubd_alloc_fn alloc;
    ubd_free_fn free;
    void *alloc_user_data;
    void *stream;           /* hipStream_t for the weight upload           */
} ubd_model_params;

typedef struct ubd_model ubd_model;

/* Load a model from the given tensors ([ENG] Steps 2-6, with host arrays
 * standing in for the GGUF file).  Every tensor the architecture needs must
 * be present exactly once with the expected shape.  Status: 0 ok; -1
 * invalid (missing, duplicate, unknown or mis-shaped tensor, mixed matrix
 * types, unsupported sizes: n_embd, n_head*head_dim, n_ff and n_vocab must
 * be multiples of 16, head_dim must be 32, 64 or 128, n_head / n_head_kv
 * at most 32, and each fused matrix (Q|K|V, gate|up, O, down, output) at
 * most 2 GiB); -2 allocation or
 * HIP failure.  Returns NULL on failure.  The model must outlive its
 * contexts. */
ubd_model *ubd_model_load(const ubd_hparams *hparams,
                          const ubd_tensor_src *tensors, int32_t n_tensors,
                          const ubd_model_params *params, int32_t *status);
void ubd_model_free(ubd_model *model);
/* Bytes of device memory held by the model's weights. */
size_t ubd_model_size(const ubd_model *model);

/* ------------------------------------------------------------------- GGUF */

/* GGUF files ([ENG] "GGUF format" reference and Steps 2-4; loading page
 * "Model loading": header parsed without tensor data, a name -> location
 * map, data mapped or read, split files).  The layout is the pages': magic
 * "GGUF", version (only 3 is read; others are rejected), tensor count, key
 * count (u64 each); key/value pairs (key string, u32 value type, value;
 * arrays: u32 element type, u64 count, elements); tensor records (name,
 * u32 n_dims <= 4, u64 sizes innermost first, u32 tensor type, u64 offset
 * from the data block); the data block.  The pages give no codes or
 * alignment; these are the public GGUF specification's:
 *   value types  0 u8, 1 i8, 2 u16, 3 i16, 4 u32, 5 i32, 6 f32, 7 bool,
 *                8 string (u64 length + bytes), 9 array, 10 u64, 11 i64,
 *                12 f64
 *   tensor types 0 F32, 1 F16, 8 Q8_0 (34-byte blocks), 30 BF16; others
 *                are rejected
 *   alignment    general.alignment (u32) or 32: the data block starts at
 *                the first multiple after the records; offsets are
 *                multiples of it.
 * Every size, count and offset is checked against the file: a malformed
 * file gives status -1 and a message, never a read outside it. */
typedef struct ubd_gguf ubd_gguf;
ubd_gguf *ubd_gguf_open(const char *path, int32_t *status);
void ubd_gguf_close(ubd_gguf *g);
uint32_t ubd_gguf_version(const ubd_gguf *g);
/* Absolute file offset of the data block. */
int64_t ubd_gguf_data_offset(const ubd_gguf *g);
/* Metadata, as the pages' gguf_get_n_kv / get_key / get_kv_type /
 * find_key / get_val_*: index i in [0, n_kv); j = -1 reads a scalar, j >= 0
 * element j of an array.  get_int covers the integer types and bool,
 * get_float f32 / f64, get_str strings (*len gets the byte length; the
 * bytes are also NUL-terminated).  Nested arrays report their type and
 * count only.  Wrong type or index: -1 / NULL. */
int64_t ubd_gguf_n_kv(const ubd_gguf *g);
int64_t ubd_gguf_find_key(const ubd_gguf *g, const char *key);
const char *ubd_gguf_key(const ubd_gguf *g, int64_t i);
int32_t ubd_gguf_kv_type(const ubd_gguf *g, int64_t i);
int32_t ubd_gguf_arr_type(const ubd_gguf *g, int64_t i);
int64_t ubd_gguf_arr_n(const ubd_gguf *g, int64_t i);
int32_t ubd_gguf_get_int(const ubd_gguf *g, int64_t i, int64_t j, int64_t *out);
int32_t ubd_gguf_get_float(const ubd_gguf *g, int64_t i, int64_t j, double *out);
const char *ubd_gguf_get_str(const ubd_gguf *g, int64_t i, int64_t j, uint64_t *len);
/* Tensor records: dims writes ne[4] (unused = 1) and returns n_dims;
 * offset is absolute in the file; nbytes from the type's block size. */
int64_t ubd_gguf_n_tensors(const ubd_gguf *g);
int64_t ubd_gguf_find_tensor(const ubd_gguf *g, const char *name);
const char *ubd_gguf_tensor_name(const ubd_gguf *g, int64_t i);
int32_t ubd_gguf_tensor_type(const ubd_gguf *g, int64_t i);
int32_t ubd_gguf_tensor_dims(const ubd_gguf *g, int64_t i, int64_t *ne);
int64_t ubd_gguf_tensor_offset(const ubd_gguf *g, int64_t i);
int64_t ubd_gguf_tensor_nbytes(const ubd_gguf *g, int64_t i);

/* Summary of a model file ([ARCH] Example 8 print_info): parameters from
 * the tensor shapes, bits per weight = file bits / parameters, the most
 * common tensor type (all_same = every tensor has it), the hyperparameters
 * as ubd_model_load_gguf reads them. */
typedef struct ubd_gguf_info {
    uint32_t version;
    int32_t n_files;
    int64_t n_tensors;
    double n_params;
    double file_bytes;
    double bpw;
    int32_t file_type;
    int32_t all_same;
    ubd_hparams hparams;
} ubd_gguf_info;
int32_t ubd_gguf_model_info(const char *path, ubd_gguf_info *info);

/* Load a llama model from a GGUF file ([ENG] Steps 2-6).  Architecture
 * general.architecture = "llama"; hyperparameters from llama.block_count,
 * .embedding_length, .feed_forward_length, .attention.head_count,
 * .attention.head_count_kv (default head_count), .context_length,
 * .attention.layer_norm_rms_epsilon, .rope.freq_base (default 10000);
 * n_vocab from token_embd.weight.  A first part named
 * <prefix>-00001-of-0000N.gguf with split.count = N pulls in the other
 * parts by name (each must carry its split.no); all tensors go into one
 * map, a name seen twice is an error.  use_mmap != 0 maps the files and
 * uploads from the mapping; 0 reads each tensor with pread.  Tensors are
 * then loaded as by ubd_model_load (same rules and status codes); the
 * print_info summary goes to the log. */
ubd_model *ubd_model_load_gguf(const char *path, const ubd_model_params *params, int32_t use_mmap,
                               int32_t *status);

/* ---------------------------------------------------------------- context */

/* Abort callback: polled before every ubatch; returning true stops the
 * decode with UBD_ABORTED ([ENG] Steps 11-12). */
typedef bool (*ubd_abort_fn)(void *user_data);

/* Context parameters ([ENG] Step 7; [DEC] "Context construction"). */
typedef struct ubd_context_params {
    uint32_t n_ctx;          /* KV cells in total; 0 = n_ctx_train; padded
                                up to a multiple of 256                    */
    uint32_t n_batch;        /* most tokens per ubd_decode call            */
    uint32_t n_ubatch;       /* most tokens per forward pass               */
    uint32_t n_seq_max;      /* sequences; 1..UBD_MAX_SEQ                  */
    ubd_type type_k;         /* K cache type: F32, F16 or Q8_0             */
    ubd_type type_v;         /* V cache type: F32, F16 or Q8_0 (Q8_0 for
                                both or neither; [ARCH] Ex. 10: 34 bytes
                                per 32 values, blocks of 32 along each
                                head's dims, scale = block max / 127)      */
    bool kv_unified;         /* false: one stream of n_ctx/n_seq_max cells
                                per sequence; true: one shared stream      */
    ubd_abort_fn abort_callback;
    void *abort_user_data;
    void *stream;            /* hipStream_t for all work; NULL = null stream */
    bool graph_reuse;        /* true (default): the first ubatch of a shape
                                is captured as a HIP graph, and later
                                ubatches of that shape replay it instead of
                                launching kernel by kernel (the graph reuse
                                of [ENG] Step 13a; [ARCH] Example 15).  The
                                shape: tokens, output rows, attention tiles
                                and, for ubatches of <= 16 tokens, the scan
                                length rounded up to 256 cells.  Bypassed
                                while kernel timing or residual keeping is
                                on; at most 16 shapes kept, least recently
                                used first out; results bit-identical to
                                graph_reuse = false                         */
} ubd_context_params;

/* n_ctx 0, n_batch 2048, n_ubatch 512, n_seq_max 1, F16/F16, not unified. */
ubd_context_params ubd_context_default_params(void);

typedef struct ubd_context ubd_context;

/* Create a context: KV cache for all cells and worst-case per-ubatch
 * buffers are allocated here ([ENG] Step 7; [ARCH] Example 10).
 * n_batch is clamped to n_ctx and n_ubatch to n_batch.  Status: 0 ok,
 * -1 invalid parameters, -2 allocation failure.  NULL on failure. */
ubd_context *ubd_init_from_model(ubd_model *model,
                                 const ubd_context_params *params,
                                 int32_t *status);
void ubd_free(ubd_context *ctx);
uint32_t ubd_n_ctx(const ubd_context *ctx);      /* padded total cells   */
uint32_t ubd_n_batch(const ubd_context *ctx);
uint32_t ubd_n_ubatch(const ubd_context *ctx);

/* ------------------------------------------------------------------ batch */

/* Mirror of llama_batch ([ENG] Step 10).  Arrays have n_tokens entries and
 * belong to the caller; they are only read during ubd_decode.
 *   token     token ids in [0, n_vocab)
 *   embd      must be NULL (token input only)
 *   pos       NULL = continue the token's first sequence from its
 *             seq_pos_max + 1; given positions must continue every
 *             sequence of the token (an empty sequence may start anywhere)
 *   n_seq_id  NULL = one sequence per token; else n_seq_id[i] >= 1
 *             distinct sequences seq_id[i][0 .. n_seq_id[i]) per token
 *             ([ENG] Step 10: a token can belong to several sequences).
 *             More than one needs a unified KV cache: the token is stored
 *             once, in one cell shared by all its sequences, and its query
 *             attends to the cells of its first sequence
 *   seq_id    NULL = sequence 0; else ids in [0, n_seq_max)
 *   logits    NULL = only the last token outputs; else nonzero = output */
typedef struct ubd_batch {
    int32_t n_tokens;
    ubd_token *token;
    float *embd;
    ubd_pos *pos;
    int32_t *n_seq_id;
    ubd_seq_id **seq_id;
    int8_t *logits;
} ubd_batch;

/* Allocate a batch with room for n_tokens_alloc tokens and n_seq_max
 * sequence ids per token (embd must be 0).  Free with ubd_batch_free. */
ubd_batch ubd_batch_init(int32_t n_tokens_alloc, int32_t embd, int32_t n_seq_max);
void ubd_batch_free(ubd_batch batch);
/* Wrap existing token ids; pos, seq_id and logits stay NULL ([ENG] Step 10). */
ubd_batch ubd_batch_get_one(ubd_token *tokens, int32_t n_tokens);

/* ----------------------------------------------------------------- decode */

/* Run one batch ([ENG] Steps 11-13; [DEC] "Batch pipeline" and
 * "process_ubatch"): validate and autofill, split into ubatches (simple
 * split with one KV stream, equal split with several), find KV cells for
 * every ubatch before committing any, then per ubatch commit its cells and
 * enqueue the forward pass.  Returns UBD_OK, UBD_NO_KV_SLOT (nothing
 * changed), UBD_ABORTED (ubatches before the aborted one are kept),
 * UBD_INVALID (nothing changed), UBD_ALLOC_FAILED or UBD_COMPUTE_FAILED
 * (the failing ubatch is removed again with seq_rm(s, pos_min, -1)).
 * Returns before the GPU finishes. */
int32_t ubd_decode(ubd_context *ctx, ubd_batch batch);

/* Number of output rows of the last successful decode (flagged tokens). */
int32_t ubd_n_outputs(const ubd_context *ctx);

/* Logits of the last decode as host f32 rows [n_outputs][n_vocab] in batch
 * order of the flagged tokens ([ENG] Step 14).  Synchronises.  Valid until
 * the next ubd_decode or ubd_free.  NULL if there are none. */
float *ubd_get_logits(ubd_context *ctx);
/* One row: i >= 0 is a batch index (NULL if that token was not flagged);
 * i < 0 counts rows from the end ([ENG] Step 14, output row lookup). */
float *ubd_get_logits_ith(ubd_context *ctx, int32_t i);
/* Device pointer to the same rows (f32, row stride n_vocab), for callers
 * that keep the data on the GPU.  Does not synchronise. */
const float *ubd_get_logits_device(ubd_context *ctx);

/* Greedy pick: the token with the largest logit, lowest id on ties
 * ([ENG] Steps 14-16, sampling).  Runs on the GPU; i as in
 * ubd_get_logits_ith.  Returns -1 for an invalid i. */
ubd_token ubd_sample_greedy(ubd_context *ctx, int32_t i);
/* Greedy pick for every output row at once: out[r] for r < n_outputs.
 * Returns the number of rows written, or -1. */
int32_t ubd_sample_greedy_all(ubd_context *ctx, ubd_token *out, int32_t cap);

/* Greedy generation of one sequence without a host round trip per token
 * ([ENG] Steps 10-16 repeated: decode one token, pick the largest logit,
 * feed it back).  Step i decodes one token of seq_id at the next position
 * (autofilled), with logits; its token is `first` for i = 0 and the pick of
 * step i-1 after that, and out[i] receives its pick (lowest id on ties, as
 * ubd_sample_greedy).  Each pick is written by the GPU straight into the
 * next step's token table, so the host plans and enqueues step i+1 while
 * step i runs; results equal ubd_decode + ubd_sample_greedy step by step.
 * The picks come back every UBD_GREEDY_CHAIN_BLOCK steps (one
 * synchronisation each).  out: host int32 [n_steps].
 * Returns the number of steps done (n_steps, or fewer when a step fails:
 * the error is then in ubd_last_error and the steps before it are kept), or
 * UBD_INVALID / a decode error code when no step was done. */
#define UBD_GREEDY_CHAIN_BLOCK 256
int32_t ubd_greedy_chain(ubd_context *ctx, ubd_token first, ubd_seq_id seq_id, int32_t n_steps, ubd_token *out);

/* The greedy pick of ubd_sample_greedy_all over caller-owned rows, for
 * callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the call allocates nothing.  Its
 * partial results live in a fixed device array of the library (one per GPU,
 * UBD_GREEDY_STATIC_MAX_ROWS rows, 128 KiB, held until the process ends);
 * each call overwrites it, so calls that overlap on one GPU (two streams, or
 * two host threads) race and must be ordered by the caller.
 *   device  : HIP device ordinal of the rows, the output and the stream
 *   logits  : device f32 rows [n_rows][ld], 16-byte aligned, read only
 *   ld      : row stride in floats, a multiple of 4, >= n_vocab
 *   n_rows  : 0 .. UBD_GREEDY_STATIC_MAX_ROWS
 *   n_vocab : values per row, a positive multiple of 4
 *   out     : device int32 [n_rows]: the largest value's index per row,
 *             the lowest index on ties
 *   stream  : hipStream_t on `device` (NULL = the null stream); the work is
 *             enqueued there and the call returns before it finishes
 * Returns UBD_OK, UBD_INVALID (arguments out of range, nothing enqueued) or
 * UBD_COMPUTE_FAILED (HIP error). */
#define UBD_GREEDY_STATIC_MAX_ROWS 256
int32_t ubd_greedy_rows_static(int32_t device, const float *logits, int32_t ld, int32_t n_rows,
                               int32_t n_vocab, ubd_token *out, void *stream);

/* Sampler chain ([ENG] Steps 14-16, "Sampler chain"): penalties of the
 * tokens already chosen, then the top-k, top-p and min-p cut-offs, then
 * temperature, then one random token.  Readings where the page gives no
 * formula:
 *   - penalties act on the distinct tokens of the last penalty_last_n
 *     history entries, count c: logit / repeat if logit > 0 else logit *
 *     repeat, then minus c * freq and minus present;
 *   - candidates are ordered by logit descending, ties by lower id;
 *   - top_k (1 .. 1024) keeps the first top_k;
 *   - top_p < 1 keeps the shortest prefix whose softmax mass (temperature
 *     1) reaches top_p;
 *   - min_p > 0 keeps probabilities >= min_p times the largest;
 *   - temperature > 0 divides the logits (<= 0: the first candidate);
 *   - the draw takes u in [0, 1) and returns the first candidate whose
 *     accumulated probability exceeds u.
 * The sampler keeps its own history, like the pages' chain: every sampled
 * token is appended, and ubd_sampler_accept appends others (a prompt). */
typedef struct ubd_sampler_params {
    int32_t top_k;           /* 1 .. 1024                                   */
    float top_p;             /* (0, 1]; 1 = off                             */
    float min_p;             /* [0, 1); 0 = off                             */
    float temperature;       /* > 0; <= 0 picks the largest logit           */
    int32_t penalty_last_n;  /* 0 .. 256 history entries penalised; 0 = off */
    float penalty_repeat;    /* 1 = off                                     */
    float penalty_freq;      /* 0 = off                                     */
    float penalty_present;   /* 0 = off                                     */
} ubd_sampler_params;
typedef struct ubd_sampler ubd_sampler;

/* top_k 40, top_p 1, min_p 0, temperature 1, no penalties. */
ubd_sampler_params ubd_sampler_default_params(void);
/* A sampler for rows of ctx's logits; device buffers on ctx's device.
 * NULL (see ubd_last_error) for parameters out of range. */
ubd_sampler *ubd_sampler_init(ubd_context *ctx, ubd_sampler_params params);
/* Frees the sampler's buffers; valid before or after its context is freed. */
void ubd_sampler_free(ubd_sampler *smpl);
/* Append a token to the sampler's history. */
void ubd_sampler_accept(ubd_sampler *smpl, ubd_token token);
/* Run the chain on logits row i (as in ubd_get_logits_ith) of the
 * sampler's context, draw with u in [0, 1), append the token to the
 * history and return it; -1 for an invalid i or u.  Synchronises. */
ubd_token ubd_sampler_sample(ubd_sampler *smpl, int32_t i, float u);
/* The same chain on a caller's row of n_vocab float logits in device
 * memory of the sampler's device (ordered on the context's stream, read
 * only).  Appends the token to the history; -1 for invalid arguments. */
ubd_token ubd_sampler_sample_logits(ubd_sampler *smpl, const float *logits, int32_t n_vocab, float u);
/* The candidates the last sample drew from, in order, with their
 * probabilities: writes min(n, cap) and returns n, the count. */
int32_t ubd_sampler_candidates(ubd_sampler *smpl, ubd_token *ids, float *probs, int32_t cap);

/* Wait for all work enqueued on the context's stream.  0 or -3. */
int32_t ubd_synchronize(ubd_context *ctx);

/* ----------------------------------------------------------------- memory */

/* Smallest / largest position held for sequence s; -1 if none
 * ([ENG] KV-cache section, seq_pos_max). */
ubd_pos ubd_memory_seq_pos_min(ubd_context *ctx, ubd_seq_id s);
ubd_pos ubd_memory_seq_pos_max(ubd_context *ctx, ubd_seq_id s);
/* Take sequence s (all sequences if s < 0) out of the cells with
 * p0 <= pos < p1; p0 < 0 means 0, p1 < 0 means infinity ([DEC] "Error
 * recovery and state rollback").  A cell that no sequence holds any more
 * is free ([DEC] "KV cache details": cells hold a set of sequences).
 * Returns false for s >= n_seq_max, else true. */
bool ubd_memory_seq_rm(ubd_context *ctx, ubd_seq_id s, ubd_pos p0, ubd_pos p1);
/* Give sequence dst the cells of src with p0 <= pos < p1 (same ranges as
 * seq_rm).  In a unified cache the cells become shared: no K/V moves.
 * With one stream per sequence only the whole sequence can be copied
 * (p0 < 0 and p1 < 0): dst's stream is replaced by a copy of src's, K/V
 * rows included.  The caller normally empties dst first; cells dst already
 * holds stay.  False for invalid ids or a partial range across streams. */
bool ubd_memory_seq_cp(ubd_context *ctx, ubd_seq_id src, ubd_seq_id dst, ubd_pos p0, ubd_pos p1);
/* Drop every sequence but s from every cell.  False for an invalid s. */
bool ubd_memory_seq_keep(ubd_context *ctx, ubd_seq_id s);
/* Defrag ([DEC] "KV cache details", defrag and its figure): in every
 * stream the occupied cells move to the lowest indices, ordered by (lowest
 * sequence of the cell, position, old index), K/V rows with them (stored
 * values unchanged), so attention scans fewer cells.  ubd_decode does the
 * same once by itself when a batch finds no free cells, then searches
 * again.  Returns the number of cells that moved, or a negative error
 * code (then the cache is unchanged).  Cells reported by ubd_get_kv_cells
 * for an earlier decode no longer apply. */
int32_t ubd_memory_defrag(ubd_context *ctx);
/* Cell table of a stream: pos[c] (-1 = empty) for its cells and, if
 * seq_words is not NULL, the sequence bits: bit (s % 32) of
 * seq_words[(s / 32) * n_cells + c] is set when cell c holds sequence s
 * (n_cells * ceil(n_seq_max / 32) words).  Returns n_cells, -1 if cap (in
 * entries of each array) is too small or the stream is invalid. */
int32_t ubd_memory_cells(ubd_context *ctx, int32_t stream, int32_t *pos, uint32_t *seq_words, int32_t cap);
/* KV cell of each batch token of the last successful decode, in batch
 * order ([DEC] "KV cache details": slot_info indices).  Returns the token
 * count, or -1 if cap is too small. */
int32_t ubd_get_kv_cells(ubd_context *ctx, int32_t *cells_out, int32_t cap);

/* Fill positions 0..n_pos-1 of the empty sequence s with given K/V rows:
 * k_layers[l] / v_layers[l] point to [n_pos][n_head_kv * head_dim] values of
 * src_type (F16 or F32; converted to the cache types, Q8_0 caches
 * quantised block by block as at append), host unless on_device.  Used to start from a long pre-filled context.  Returns 0,
 * UBD_NO_KV_SLOT if the stream lacks room, UBD_INVALID otherwise. */
int32_t ubd_kv_fill(ubd_context *ctx, ubd_seq_id s, int32_t n_pos,
                    const void *const *k_layers, const void *const *v_layers,
                    ubd_type src_type, int32_t on_device);
/* Read back the K (which = 0) or V (which = 1) rows of cells
 * [cell0, cell0 + n) of one layer and KV stream as f32
 * [n][n_head_kv * head_dim] into host memory (Q8_0: f16(scale) * code).
 * Synchronises.  0 or -1. */
int32_t ubd_kv_read(ubd_context *ctx, int32_t layer, int32_t stream,
                    int32_t which, int32_t cell0, int32_t n, float *out);

/* ------------------------------------------------------- diagnostics/perf */

/* Keep the residual stream entering every layer (and after the last) for
 * the most recent ubatch, like the pages' per-node eval callback
 * ([ARCH] Example 4).  enable = 0 frees it.  0 or -2. */
int32_t ubd_debug_keep_residuals(ubd_context *ctx, int32_t enable);
/* Copy the kept residual entering layer `layer` (layer == n_layer: after
 * the last layer) for the n_tokens tokens of the last ubatch, in ubatch
 * order, as f32 [n_tokens][n_embd].  Synchronises.  Returns the token count
 * or -1. */
int32_t ubd_debug_get_residual(ubd_context *ctx, int32_t layer, float *out,
                               int32_t cap_tokens);
/* Batch index of every token of the last ubatch, in ubatch order. */
int32_t ubd_debug_last_ubatch(ubd_context *ctx, int32_t *batch_idx,
                              int32_t cap);

/* Kernel timing with HIP events tied to the kernel dispatches (the first
 * kernel of a timed launch records its start, the last its end, so a
 * launch's interval is its kernels' execution without their dispatch, the
 * durations a kernel trace reports).  Kernels fall in
 * classes 2*kind + phase, phase 0 for ubatches of <= 16 tokens (decode) and
 * 1 for larger ones (prefill), kind 0 embed, 1 rmsnorm, 2 qkv (+RoPE and
 * K/V append), 3 attention (partial + combine), 4 attn_output (+residual),
 * 5 ffn_gate_up (+SwiGLU), 6 ffn_down (+residual), 7 logits.  mask selects
 * the timed classes (bit = class); 0 turns timing off.  0 or -1. */
#define UBD_KERNEL_CLASSES 16
int32_t ubd_debug_kernel_timing(ubd_context *ctx, uint32_t mask);
/* Name of a class, e.g. "decode.ffn_gate_up"; "" for an invalid class. */
const char *ubd_debug_kernel_class_name(int32_t cls);
/* Synchronises, then writes the launches and summed milliseconds of the
 * first n classes since the last call and resets them.  n or -1. */
int32_t ubd_debug_kernel_stats(ubd_context *ctx, int32_t *launches,
                               double *total_ms, int32_t n);

/* Process-wide launch-shape knobs for measurements: "skinny_nw" (waves
 * per work-group of the few-token products: 4, 8, 16; 0 = automatic),
 * "fuse_norm" (ubatches of at most 2 tokens: 1 = RMSNorm fused into the
 * QKV, gate|up and logits products, -1 = into QKV only, 0 = never),
 * "attn_chunk_min" (smallest cells per wave of split attention, default
 * 64, at least 32), "attn_pair" (prefill attention: 1 = two waves per
 * tile, each scanning half its cells, 0 = one wave), "attn_nt_mb"
 * (split attention that streams at least this many MB of K/V per launch
 * loads it non-temporally; default 32, -1 = never), "ldsx"
 * (0 = few-token products read activations from global memory),
 * "ldsx_early" (one-token products: 1 = activation loads issued before the
 * weight loads, 0 = after; the results are identical), "gemm_wpd"
 * (prefill product weight look-ahead stages, 1 or 2; 0 = per shape),
 * "gemm_deep" (1 = bf16 residual and QKV prefill products use the kernel
 * with weights three stages ahead where the shape allows, 0 = never),
 * "act_tiled" (1 = the prefill products read their input activations
 * stored in matrix-core operand order, 0 = row-major), "gemm"
 * (prefill products: 1 = LDS-ring kernel, 0 = register-staged kernel),
 * "gemm_shape" (0 = automatic LDS-ring tile; 1, 2, 3, 4 force 2x4, 2x8,
 * 4x4, 4x8 blocks of 16 weight rows per wave x 16 tokens; 5, 6 force 1x4,
 * 1x8 for products without SwiGLU; bf16 weights with the weights loaded
 * further ahead in rotating register sets, where K / 64 is a multiple of
 * the set count: 7 = 4x8 one stage ahead and 8 = 4x8 three stages ahead
 * with one wave per SIMD, 9 = 2x8, 10 = 2x4, 11 = 4x4 three stages ahead,
 * 12 = 4x16 one stage ahead with one wave per SIMD; three stages ahead
 * with residual products split in two over k through scratch: 13 = 4x4,
 * 14 = 2x4, 15 = 2x8; with both activation planes, 4x4 one stage ahead: 16
 * unsplit, 18 with residual products in two k slices, 19 in four; 20 = 2x4
 * three stages ahead with the activations three stages ahead, the residual
 * short-k products' automatic tile; 21 = the wide 256 x 128 tile of 8 waves
 * with weights and activations staged in LDS, 22 the same with residual
 * products in four k slices, 23 the same unsplit with a 2-deep ring, two
 * work-groups per CU; 24 = the wide kernel's 128 x 64 tile, 8 waves of
 * 32 x 32, 25 the same with residual products in two k slices),
 * "gemm_split"
 * (residual prefill products: 0 = automatic k split, 2 or 4 forced),
 * "small_rb" (1 =
 * products of 3..16 tokens share activation fragments over 4 row blocks
 * or split k, 0 = one row block per work-group), "prefill_lo" (bf16
 * prefill products whose activations enter the matrix cores as hi and lo
 * bf16 planes, a mask of bits 1 QKV, 2 O, 4 gate|up, 8 down, 16 logits;
 * default 31 = all; the others take the hi plane only, i.e. bf16-rounded
 * activations, which leaves about 6e-3 of relative error per 8B-shaped
 * layer; with both planes the forced shapes are 1, 3, 5, 10, 14, 16 and 18
 * to 25), "post_norm" (1 = a residual prefill product whose k is split
 * runs the RMSNorm that follows it in the pass adding its k slices, 0 =
 * the norm in its own kernel; the results are identical).
 * Results do not depend on them beyond rounding, except "prefill_lo".
 * The knobs are process-wide and unsynchronised: set them while no other
 * thread is inside the library; every context sees the change.  0, or -1
 * for an unknown key. */
int32_t ubd_debug_set_tuning(const char *key, int32_t value);

/* Counters in the spirit of llama_perf_context_print ([ARCH] Example 15). */
typedef struct ubd_perf {
    double t_load_ms;       /* ubd_model_load wall time                    */
    double t_p_eval_ms;     /* host time in ubd_decode, batches > 1 token  */
    double t_eval_ms;       /* host time in ubd_decode, 1-token batches    */
    int32_t n_p_eval;       /* tokens in batches > 1 token                 */
    int32_t n_eval;         /* 1-token batches                             */
    int32_t n_ubatch;       /* forward passes enqueued                     */
    int32_t n_decode;       /* ubd_decode calls returning UBD_OK           */
    int32_t n_graphs;       /* ubatch graphs captured                      */
    int32_t n_reused;       /* ubatches that replayed a captured graph
                               (the reuse count of [ARCH] Example 15's
                               timing summary)                             */
} ubd_perf;
void ubd_perf_get(const ubd_context *ctx, ubd_perf *out);
void ubd_perf_reset(ubd_context *ctx);

/* Log sink for info and error lines; NULL restores stderr for errors. */
typedef void (*ubd_log_fn)(int32_t level, const char *text, void *user_data);
void ubd_log_set(ubd_log_fn fn, void *user_data);
/* Message of the last failure on this thread ("" if none). */
const char *ubd_last_error(void);

/* ---------------------------------------------------- host-only planner */

/* The batch/ubatch/KV-cell bookkeeping of ubd_decode without a GPU: the
 * same code ubd_decode runs, with the forward pass replaced by a stub that
 * succeeds, or returns fail_code (UBD_ABORTED or UBD_COMPUTE_FAILED) at
 * ubatch fail_at (fail_at < 0: never).  n_ctx, n_batch, n_ubatch,
 * n_seq_max and kv_unified as in ubd_context_params. */
typedef struct ubd_planner ubd_planner;
ubd_planner *ubd_planner_new(uint32_t n_ctx, uint32_t n_batch,
                             uint32_t n_ubatch, uint32_t n_seq_max,
                             bool kv_unified, int32_t n_vocab);
void ubd_planner_free(ubd_planner *p);
int32_t ubd_planner_decode(ubd_planner *p, ubd_batch batch, int32_t fail_at,
                           int32_t fail_code);
/* Ubatches of the last decode and, for ubatch k, its tokens' batch
 * indices, cells and streams (arrays of at least its token count). */
int32_t ubd_planner_n_ubatches(const ubd_planner *p);
int32_t ubd_planner_ubatch(const ubd_planner *p, int32_t k, int32_t *batch_idx,
                           int32_t *cells, int32_t *streams, int32_t cap);
/* Output row of batch index i (-1 if none) and the row count. */
int32_t ubd_planner_output_row(const ubd_planner *p, int32_t i);
int32_t ubd_planner_n_outputs(const ubd_planner *p);
ubd_pos ubd_planner_seq_pos_min(const ubd_planner *p, ubd_seq_id s);
ubd_pos ubd_planner_seq_pos_max(const ubd_planner *p, ubd_seq_id s);
bool ubd_planner_seq_rm(ubd_planner *p, ubd_seq_id s, ubd_pos p0, ubd_pos p1);
bool ubd_planner_seq_cp(ubd_planner *p, ubd_seq_id src, ubd_seq_id dst, ubd_pos p0, ubd_pos p1);
bool ubd_planner_seq_keep(ubd_planner *p, ubd_seq_id s);
int32_t ubd_planner_defrag(ubd_planner *p);
int32_t ubd_planner_cells(const ubd_planner *p, int32_t stream, int32_t *pos, uint32_t *seq_words, int32_t cap);
/* Cells scanned by attention in a stream: highest used cell + 1. */
int32_t ubd_planner_n_kv(const ubd_planner *p, int32_t stream);

#ifdef __cplusplus
}
#endif

#endif /* UBD_H */
