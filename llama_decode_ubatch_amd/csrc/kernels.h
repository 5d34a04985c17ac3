// Host-callable launchers of the gfx950 kernels (kernels.hip).
//
// Layouts shared by the kernels and the runtime:
//  * Activations are row-major [tokens][features].  An activation given to
//    a matrix product is either F32 (f32 weights) or HILO: two bf16 planes
//    with x ~= hi + lo (hi = bf16(x), lo = bf16(x - hi)), which keeps about
//    16 significand bits when the weights are bf16 or q8_0.
//  * Weight matrices [rows][cols] are stored pre-tiled in MFMA fragment
//    order: one 1 KB tile per 16-row block and k-step, lane l = 16*g + r
//    holding 16 bytes of row r:
//      f32 : k-step 16 values, lane bytes = cols 16*s + 4g .. +4
//      bf16: k-step 32 values, lane bytes = cols 32*s + 8g .. +8
//      q8_0: k-step 64 values, lane bytes = cols 64*s + 8g .. +8 then
//            cols 64*s + 32 + 8g .. +8 (codes), scales as
//            [row block][cols/32][16 rows] f16.
//    Tiles are stored k-step-major: tile (rb, s) starts at byte
//    (s * rows/16 + rb) * 1024, so that the work-groups of a product, which
//    advance through k together, read one contiguous window of memory.
//  * KV cache per layer: K [stream][kv head][cell][head_dim] and V in
//    32-cell tiles [stream][kv head][cell / 32][head_dim][32], each of
//    type_k / type_v (q8_0: int8 codes in these layouts, then the f16 block
//    scales, see kv_layer_bytes).  n_cells given to the kernels is the per-stream cell
//    stride, the context's cells per stream rounded up to 32; the device
//    cell tables [stream][n_cells] hold pos = seq = -1 in the padding.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ubd {

enum WType : int { W_F32 = 0, W_BF16 = 2, W_Q8 = 3 };

// Launch-shape knobs (process-wide; 0 = built-in choice).  Set through
// ubd_debug_set_tuning for measurements.
struct Tuning {
    int skinny_nw = 0;        // waves per work-group of the small-T product
    int fuse_norm = 1;        // ubatches of <= 2 tokens: 1 = RMSNorm fused into the QKV, gate|up and
                              // logits products, -1 = into QKV only, 0 = never
    int attn_chunk_min = 64;  // smallest cells per wave of split attention (>= 32)
    int attn_pair = 1;        // unsplit (prefill) MFMA attention: 1 = two waves per tile, each scanning half
    int attn_nt_mb = 32;      // split attention streaming >= this many MB of K/V per launch loads it
                              // non-temporally (-1 = never)
    int ldsx = 1;             // stage few-token activations in LDS (decode products)
    int ldsx_early = 1;       // one-token LDS-staged products: activation loads ahead of the weights
    int small_rb = 1;         // several-token products: 4 row blocks per work-group / split k (0 = off)
    int gemm = 1;             // prefill products: 1 = LDS-ring kernel, 0 = register-staged kernel
    int gemm_split = 0;       // residual prefill products: forced k split (2, 4; 0 = automatic)
    int gemm_shape = 0;       // LDS-ring tile (0 = automatic; 1..4 force 2x4, 2x8, 4x4, 4x8 row x token blocks)
    int gemm_wpd = 0;         // LDS-ring product: stages of weight look-ahead (1 or 2; 0 = per shape)
    int gemm_deep = 1;        // bf16 residual / QKV prefill products: 1 = deep look-ahead kernel where it fits
    int act_tiled = 1;        // prefill products read activations tiled in MFMA operand order (0 = row-major)
    int prefill_lo = 31;      // bf16 prefill products whose activations enter as hi + lo planes (two
                              // products per fragment), bit 1 << Prod; the others take the hi plane
                              // only (bf16-rounded activations)
    int post_norm = 1;        // residual products with split k: the next RMSNorm runs in the pass that
                              // adds the slices (0 = its own kernel)
};
// LDS bytes the activation copy of the LDS-staged few-token product may use
constexpr size_t LDSX_MAX_BYTES = 64 * 1024;
extern Tuning g_tuning;

// Kernel timing: while stop is set, every launch of this thread records
// stop when its kernel ends and the first one records start when its
// kernel begins (events tied to the dispatches themselves, so a timed
// region spans its kernels' execution, not their dispatch).
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchTiming g_launch_timing;
enum KVType : int { KV_F32 = 0, KV_F16 = 1, KV_Q8 = 2 };
// One layer of one cache (K or V) holding `elems` values: f32 / f16 values,
// or for q8_0 the int8 codes (in the f16 layouts) followed by one f16 scale
// per 32 values, ordered [stream][kv head][head_dim / 32][cell].
inline size_t kv_layer_bytes(int type, size_t elems) {
    return type == KV_F32 ? elems * 4 : type == KV_F16 ? elems * 2 : elems + elems / 32 * 2;
}

struct Act {
    float *f32 = nullptr;      // F32 format
    uint16_t *hi = nullptr;    // HILO format
    uint16_t *lo = nullptr;
    int ld = 0;                // elements per row
    // HILO planes in MFMA operand order instead of row-major: 1 KB tiles of
    // 16 tokens x 32 values, tile (t / 16, k / 32) at ((t / 16) * (ld / 32) +
    // k / 32) * 512 elements, value (t, k) at lane (t % 16) + 16 * ((k / 8) % 4),
    // element k % 8 of that lane's 8 (ld a multiple of 32; buffers hold whole
    // 16-token tiles)
    int tiled = 0;
};

// Per-ubatch token table on the device (int32 planes of capacity `cap`).
constexpr int MAX_SEQ_WORDS = 8;   // sequence-mask words per cell: 256 sequences

struct TokInfo {
    const int32_t *token, *pos, *seq, *stream, *cell, *out_row, *tile_of;
    const int32_t *out_tok;    // ubatch indices of output tokens
    const int32_t *tiles;      // [n_tiles][4] = t0, n_tokens, stream, n_kv
    const uint32_t *seqw;      // [token][n_seq_words] every sequence of the token
    int n_seq_words = 1;       // seq is the first of them: attention follows it
};

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV = 3, EPI_LOGITS = 4 };
// The products of a layer and the output head (bit positions of the
// prefill_lo tuning mask)
enum Prod : int { PROD_QKV = 0, PROD_O = 1, PROD_GATE_UP = 2, PROD_DOWN = 3, PROD_LOGITS = 4 };

struct QKVEpi {
    int n_q_rows = 0, n_k_rows = 0;   // H*hd, Hk*hd
    int head_dim = 0, n_head_kv = 0, n_cells = 0;
    const float2 *rope_cs = nullptr;  // [T][head_dim / 2] (cos, sin) of each token's angles
    float *q_out = nullptr;           // [T][H*hd] f32, RoPE applied
    void *k_cache = nullptr;          // layer base
    void *v_cache = nullptr;
    int type_k = KV_F16, type_v = KV_F16;
    float *kv_stage = nullptr;        // q8_0 caches: [T][2][Hk*hd] f32 K (after RoPE) and V rows,
                                      // quantised into the cells by launch_kv_quant
};

// Fused RMSNorm of the product's input (at most NORM_TMAX rows): x row of
// token t is rows ? rows[t] : t, row stride ld; output = x / sqrt(mean(x^2)
// + eps) * gain, formed per work-group in LDS.
constexpr int NORM_TMAX = 2;
struct NormIn {
    const float *x = nullptr;
    const int32_t *rows = nullptr;
    const float *gain = nullptr;
    float eps = 0.f;
    int ld = 0;
};

// RMSNorm that a residual product runs after its k slices are added (see
// LinearArgs::post): rows of the updated residual, normalised with gain and
// eps into out (tiled hi + lo planes).
struct NormOut {
    const float *gain = nullptr;
    float eps = 0.f;
    Act out;
};

struct LinearArgs {
    int wtype = W_BF16;
    const void *w = nullptr;          // tiled weights
    const uint16_t *wscale = nullptr; // q8_0 scales (tiled)
    int N = 0, K = 0;                 // rows (outputs), cols (inputs)
    Act x;                            // input [T][K] in F32 or HILO
    int T = 0;                        // tokens
    int epi = EPI_STORE;
    float *y = nullptr;               // STORE / RESID target [T][ldy]
    int ldy = 0;
    Act out;                          // SWIGLU output [T][N/2]
    const int32_t *row_map = nullptr; // LOGITS: output row of each token
    float *logits = nullptr;          // LOGITS: [rows][N]
    TokInfo tok;                      // QKV: pos / stream / cell per token
    QKVEpi qkv;
    NormIn norm;                      // set: input is x normalised on the fly (T <= 16)
    int early = 1;                    // LDS-staged product: one-token activation loads may go first
    int prod = PROD_QKV;              // which product this is (Prod)
    float *split_out = nullptr;       // RESID prefill products: scratch for k-slice partial sums,
                                      // [MAX_K_SLICES][T][N] f32 (null: no k split)
    // RESID products: when post.gain is set and the product's k is split, the
    // pass that adds the slices into y also normalises each updated row of y
    // (all T rows, N values each) into post.out (tiled planes, N <= 8192) and
    // sets *post_done; otherwise *post_done is left false and the caller runs
    // that norm itself
    NormOut post;
    bool *post_done = nullptr;
};
// Most k slices a residual prefill product is split into (its partial sums
// go to scratch and are added to the residual in slice order).
constexpr int MAX_K_SLICES = 4;

// Enqueues y = W x with the epilogue a.epi.  Returns false, launching
// nothing, when a fused norm is asked for outside linear_norm_fits.
bool launch_linear(const LinearArgs &a, hipStream_t s);
// True when a product over T input rows of K values can take its RMSNorm
// fused (a.norm): the one- and few-token products (T <= 16).
bool linear_norm_fits(int T, int K);
// True when launch_linear(a) runs a product that reads its input activations
// in the tiled layout (the LDS-ring prefill products); the producer of a.x
// must then write that layout.
bool linear_reads_tiled(const LinearArgs &a);

// x[t] = dequant(table[token[t]]); also records the position and the
// sequence mask of each token's cell in the device cell tables
// (cell_pos [stream][n_cells], cell_seq [stream][n_seq_words][n_cells]),
// and fills the ubatch's RoPE table: rope_cs[t][i] = (cos, sin) of
// pos[t] * inv_freq[i], the angle and both functions in double precision,
// rounded to f32 (i < head_dim / 2 <= 256).
void launch_embed(int wtype, const void *table, const uint16_t *scales,
                  int d, const TokInfo &ti, int T, float *x,
                  int32_t *cell_pos, uint32_t *cell_seq, int n_cells,
                  const double *inv_freq, int half_dim, float2 *rope_cs,
                  hipStream_t s);

// out[r] = rmsnorm(x[src_row(r)]) * gain, src_row = row_map ? row_map[r] : r
// (into a tiled HILO `out` too; the rows of its last tile past `rows` are
// left as they were)
void launch_rmsnorm(const float *x, int ldx, const int32_t *row_map, int rows,
                    const float *gain, int d, float eps, const Act &out,
                    hipStream_t s);

struct AttnArgs {
    const float *q = nullptr;         // [T][H*hd] f32 (RoPE applied)
    const void *k_cache = nullptr;    // layer base
    const void *v_cache = nullptr;
    int type_k = KV_F16, type_v = KV_F16;
    size_t layer_elems = 0;           // values per layer of each cache (q8_0 scale offset)
    const int32_t *cell_pos = nullptr;    // [stream][n_cells]; -1 = empty
    const uint32_t *cell_seq = nullptr;   // [stream][n_seq_words][n_cells] sequence bits
    int n_seq_words = 1;
    int n_cells = 0, n_head = 0, n_head_kv = 0, head_dim = 0;
    TokInfo tok;
    int T = 0, n_tiles = 0, max_chunks = 0;
    float *part_o = nullptr;          // [T][H][max_chunks][hd]
    float *part_ml = nullptr;         // [T][H][max_chunks][2]
    Act out;                          // [T][H*hd]
    bool split = false;               // MFMA path: split cells into chunks + combine
    int chunk_cells = 32;             // MFMA split: cells per wave (multiple of 32)
    int n_chunks_launch = 0;          // MFMA split: chunks launched per tile
    int waves = 1;                    // MFMA, not split: waves per (tile, KV head), 1 or 2
    bool kv_nt = false;               // MFMA split: K/V codes loaded non-temporally
};
constexpr int ATTN_CHUNK = 256;       // cells per split-K chunk (f32 path)
constexpr int ATTN_DECODE_CHUNK = 32; // smallest cells-per-wave chunk of the split MFMA path
constexpr int ATTN_TILE_ROWS = 64;    // query rows (tokens x n_gqa) per tile

void launch_attention(const AttnArgs &a, hipStream_t s);
// Query rows (tokens x n_gqa) one attention tile holds for a head size.
int attn_tile_rows(int head_dim);
// MFMA attention (f16 K/V): tiles are blocks of 16 / n_gqa tokens; with
// split (at most 16 tokens), tiles[3] cells are cut into chunk_cells-cell
// chunks, one wave each, merged by a combine pass; otherwise `waves` waves
// of one work-group scan tiles[3] cells and merge in LDS.  Partials are indexed with max_chunks = ceil(n_cells /
// ATTN_DECODE_CHUNK).
bool attn_mfma_ok(int type_k, int type_v, int head_dim, int n_gqa);
void launch_attention_mfma(const AttnArgs &a, hipStream_t s);

// out[r] = argmax over n of logits[row(r)][n] (lowest index on ties).
// Workspace: pv / pi [n_rows][ARGMAX_BLOCKS] and counter [n_rows], the
// counters zero before the first call (each call leaves them zero).
constexpr int ARGMAX_BLOCKS = 64;
struct ArgmaxWork {
    float *pv = nullptr;
    int32_t *pi = nullptr;
    int32_t *counter = nullptr;
};
// out2 (optional): a second destination of the picks.
void launch_argmax(const float *logits, int ld, const int32_t *rows, int n_rows,
                   int n, int32_t *out, const ArgmaxWork &w, hipStream_t s, int32_t *out2 = nullptr);
// The same argmax in two kernels and no counter (nothing to keep at zero
// between calls): pv / pi [n_rows][ARGMAX_BLOCKS] hold the slice winners.
void launch_argmax_two_pass(const float *logits, int ld, int n_rows, int n, int32_t *out,
                            float *pv, int32_t *pi, hipStream_t s);

// Sampler chain on one logits row (one work-group): penalties of the
// history tokens, top-k (1..SAMPLER_KMAX), top-p, min-p, temperature, then
// the draw with u; out_token = {chosen id, number of candidates left},
// out_ids / out_probs = those candidates in order with their final
// probabilities.
constexpr int SAMPLER_KMAX = 1024;
constexpr int SAMPLER_HMAX = 256;
struct SamplerArgs {
    const float *logits = nullptr;
    int n_vocab = 0;
    const int32_t *hist = nullptr;    // last penalty_last_n chosen tokens (<= SAMPLER_HMAX)
    int n_hist = 0;
    int top_k = 40;
    float top_p = 1.f, min_p = 0.f, temperature = 1.f;
    float pen_repeat = 1.f, pen_freq = 0.f, pen_present = 0.f;
    float u = 0.f;
    int32_t *out_token = nullptr;     // [2]
    int32_t *out_ids = nullptr;       // [SAMPLER_KMAX]
    float *out_probs = nullptr;       // [SAMPLER_KMAX]
};
void launch_sampler(const SamplerArgs &a, hipStream_t s);

// Weight relayout: row-major source matrices -> tiled layout.  Up to three
// sources are concatenated by rows (mode 0) or two are interleaved by
// 16-row blocks, block 2j from src[0], block 2j+1 from src[1] (mode 1).
struct RelayoutSrc {
    const void *data = nullptr;        // row-major [rows][K]
    const uint16_t *scales = nullptr;  // q8_0: [rows][K/32]
    int rows = 0;
};
void launch_relayout(int wtype, const RelayoutSrc *src, int n_src, int mode,
                     int K, void *dst, uint16_t *dst_scales, hipStream_t s);

// q8_0 caches: quantise KV rows [n][n_head_kv*hd] (row stride ld, src_type
// KV_F32 / KV_F16) into the cells cells[r] of streams streams[r] (or of
// `stream` when streams is null); is_v selects the V layout.  Per 32-value
// block: d = amax / 127, codes = round-half-away(x / d), scale f16(d).
void launch_kv_quant(const void *src, int src_type, int ld, int n, const int32_t *cells, const int32_t *streams,
                     int stream, void *cache, bool is_v, int n_head_kv, int hd, int n_cells, size_t layer_elems,
                     hipStream_t s);

// KV rows [n][n_head_kv*hd] of src_type (KV_F32 / KV_F16) into the cache
// cells cells[0..n) of one stream (K rows, V in 32-cell tiles).
void launch_kv_store(const void *src, int src_type, int n, const int32_t *cells,
                     void *cache, int type, bool transposed, int stream,
                     int n_head_kv, int hd, int n_cells, hipStream_t s);
// Cache rows of cells [cell0, cell0+n) of one stream as f32 [n][n_head_kv*hd].
void launch_kv_load(const void *cache, int type, bool transposed, int stream,
                    int cell0, int n, int n_head_kv, int hd, int n_cells,
                    size_t layer_elems, float *out, hipStream_t s);
// Load-time conversions: q8_0 blocks as GGUF stores them (f16 scale, then
// 32 int8 codes: 34 bytes) into code and scale planes; f16 values widened
// to f32 (exact).
void launch_q8_blocks_split(const void *blocks, size_t n_blocks, int8_t *codes, uint16_t *scales,
                            hipStream_t s);
void launch_f16_to_f32(const uint16_t *src, size_t n, float *dst, hipStream_t s);

// Bytes of tmp that kv_move needs for n cells.
size_t kv_move_tmp_bytes(int type, int n, int n_head_kv, int hd);
// Cell moves of one layer's K or V cache, stored values unchanged (q8_0
// scales included): to_tmp copies the rows of cells[m] of the stream into
// tmp row m, otherwise tmp row m into cells[m].
void launch_kv_move(void *cache, int type, bool transposed, int stream, const int32_t *cells, int n,
                    int n_head_kv, int hd, int n_cells, size_t layer_elems, void *tmp, bool to_tmp,
                    hipStream_t s);

}  // namespace ubd
