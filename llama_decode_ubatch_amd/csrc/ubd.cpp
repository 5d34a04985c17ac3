// libubd runtime: model loading, contexts, the per-ubatch kernel schedule
// and the C ABI declared in include/ubd.h.
//
// One forward pass per ubatch follows the per-layer outline of the engine
// page ("llama.cpp AI LLM Engine - how it works", Step 13b) and the decode
// node list of the architecture page ("llama.cpp Architecture", Example 4):
//   embed -> per layer [RMSNorm -> QKV product (+RoPE, +K/V append into the
//   ubatch's cells) -> attention over the stream's cells -> O product
//   (+residual) -> RMSNorm -> gate|up product (+SwiGLU) -> down product
//   (+residual)] -> output rows -> RMSNorm -> logits product.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "kernels.h"
#include "common.h"
#include "planner.h"
#include "ubd.h"

using namespace ubd;

namespace {

thread_local std::string g_err;
ubd_log_fn g_log = nullptr;
void *g_log_ud = nullptr;

void log_line(int level, const char *fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (g_log)
        g_log(level, buf, g_log_ud);
    else if (level >= 2)
        fprintf(stderr, "ubd: %s\n", buf);
}

void set_err(const std::string &m) {
    g_err = m;
    log_line(2, "%s", m.c_str());
}

// bumped by every tuning change: a captured decode-step graph holds the
// kernel choices made when it was captured
uint32_t g_tuning_gen = 0;

}  // namespace

namespace ubd {
void set_error(const std::string &msg) { set_err(msg); }
void log_msg(int level, const char *fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    log_line(level, "%s", buf);
}
}  // namespace ubd

namespace {

bool hip_ok(hipError_t e, const char *what) {
    if (e == hipSuccess) return true;
    set_err(std::string(what) + ": " + hipGetErrorString(e));
    return false;
}

double now_ms() {
    using namespace std::chrono;
    return duration<double, std::milli>(steady_clock::now().time_since_epoch()).count();
}

int wtype_of(ubd_type t) {
    switch (t) {
    case UBD_TYPE_F32: return W_F32;
    case UBD_TYPE_F16: return W_F32;      // widened exactly at load
    case UBD_TYPE_BF16: return W_BF16;
    case UBD_TYPE_Q8_0: return W_Q8;
    default: return -1;
    }
}

size_t elem_bytes(int wtype) { return wtype == W_F32 ? 4 : wtype == W_BF16 ? 2 : 1; }

int kstep_of(int wtype) { return wtype == W_F32 ? 16 : wtype == W_BF16 ? 32 : 64; }

// Device memory owner that goes through the caller's hooks (or hipMalloc).
struct DevAlloc {
    ubd_alloc_fn alloc = nullptr;
    ubd_free_fn free = nullptr;
    void *ud = nullptr;
    std::vector<void *> blocks;
    size_t bytes = 0;

    void *get(size_t n) {
        n = (n + 255) / 256 * 256;
        if (n == 0) n = 256;
        void *p = nullptr;
        if (alloc) {
            p = alloc(n, ud);
        } else if (hipMalloc(&p, n) != hipSuccess) {
            p = nullptr;
        }
        if (p) {
            blocks.push_back(p);
            bytes += n;
        }
        return p;
    }
    void release() {
        for (void *p : blocks) {
            if (free)
                free(p, ud);
            else
                (void)hipFree(p);
        }
        blocks.clear();
        bytes = 0;
    }
};

}  // namespace

struct DevMat {
    int wtype = W_F32;
    int rows = 0, cols = 0;
    void *w = nullptr;
    uint16_t *scales = nullptr;
};

struct ubd_model {
    ubd_hparams hp{};
    int device = 0;
    hipStream_t stream = nullptr;
    DevAlloc mem;
    int wtype = W_F32;
    int head_dim = 0;
    void *embd = nullptr;
    uint16_t *embd_scales = nullptr;
    struct Layer {
        float *attn_norm = nullptr, *ffn_norm = nullptr;
        DevMat qkv, o, gu, down;
    };
    std::vector<Layer> layers;
    float *out_norm = nullptr;
    DevMat out;
    double t_load_ms = 0;
};

// -------------------------------------------------------------- model load
namespace {

struct Expect {
    int64_t ne0, ne1;
    bool gain;
};

std::map<std::string, Expect> expected_tensors(const ubd_hparams &hp) {
    const int64_t d = hp.n_embd, hd = hp.n_embd / hp.n_head;
    const int64_t nq = hd * hp.n_head, nk = hd * hp.n_head_kv;
    std::map<std::string, Expect> m;
    m["token_embd.weight"] = {d, hp.n_vocab, false};
    m["output_norm.weight"] = {d, 1, true};
    m["output.weight"] = {d, hp.n_vocab, false};
    for (int il = 0; il < hp.n_layer; ++il) {
        const std::string p = "blk." + std::to_string(il) + ".";
        m[p + "attn_norm.weight"] = {d, 1, true};
        m[p + "attn_q.weight"] = {d, nq, false};
        m[p + "attn_k.weight"] = {d, nk, false};
        m[p + "attn_v.weight"] = {d, nk, false};
        m[p + "attn_output.weight"] = {nq, d, false};
        m[p + "ffn_norm.weight"] = {d, 1, true};
        m[p + "ffn_gate.weight"] = {d, hp.n_ff, false};
        m[p + "ffn_up.weight"] = {d, hp.n_ff, false};
        m[p + "ffn_down.weight"] = {hp.n_ff, d, false};
    }
    return m;
}

// Copies a source tensor to device memory if it lives on the host.
struct Staged {
    Staged() = default;
    Staged(const Staged &) = delete;
    Staged &operator=(const Staged &) = delete;
    const void *data = nullptr;
    const uint16_t *scales = nullptr;
    std::vector<void *> tmp;
    ~Staged() {
        for (void *p : tmp) (void)hipFree(p);
    }
};

bool stage(const ubd_tensor_src &s, int wtype, hipStream_t st, Staged *out) {
    const size_t n = (size_t)s.ne[0] * s.ne[1];
    // sources that need a conversion pass on the device first
    const bool q8_blocks = s.type == UBD_TYPE_Q8_0 && !s.scales;
    if (q8_blocks || s.type == UBD_TYPE_F16) {
        const size_t in_bytes = q8_blocks ? n / 32 * 34 : n * 2;
        const void *in = s.data;
        if (!s.on_device) {
            void *d = nullptr;
            if (!hip_ok(hipMalloc(&d, in_bytes), "staging allocation")) return false;
            out->tmp.push_back(d);
            if (!hip_ok(hipMemcpyAsync(d, s.data, in_bytes, hipMemcpyHostToDevice, st), "weight upload")) return false;
            in = d;
        }
        void *a = nullptr, *b = nullptr;
        if (q8_blocks) {
            if (!hip_ok(hipMalloc(&a, n), "staging allocation")) return false;
            out->tmp.push_back(a);
            if (!hip_ok(hipMalloc(&b, n / 32 * 2), "staging allocation")) return false;
            out->tmp.push_back(b);
            launch_q8_blocks_split(in, n / 32, (int8_t *)a, (uint16_t *)b, st);
            out->scales = (const uint16_t *)b;
        } else {
            if (!hip_ok(hipMalloc(&a, n * 4), "staging allocation")) return false;
            out->tmp.push_back(a);
            launch_f16_to_f32((const uint16_t *)in, n, (float *)a, st);
        }
        out->data = a;
        return hip_ok(hipGetLastError(), "weight conversion");
    }
    const size_t bytes = n * (wtype < 0 ? 4 : elem_bytes(wtype));
    const size_t sbytes = wtype == W_Q8 ? (n / 32) * 2 : 0;
    if (s.on_device) {
        out->data = s.data;
        out->scales = (const uint16_t *)s.scales;
        return true;
    }
    void *d = nullptr;
    if (!hip_ok(hipMalloc(&d, bytes), "staging allocation")) return false;
    out->tmp.push_back(d);
    if (!hip_ok(hipMemcpyAsync(d, s.data, bytes, hipMemcpyHostToDevice, st), "weight upload")) return false;
    out->data = d;
    if (sbytes) {
        void *sd = nullptr;
        if (!hip_ok(hipMalloc(&sd, sbytes), "staging allocation")) return false;
        out->tmp.push_back(sd);
        if (!hip_ok(hipMemcpyAsync(sd, s.scales, sbytes, hipMemcpyHostToDevice, st), "scale upload")) return false;
        out->scales = (const uint16_t *)sd;
    }
    return true;
}

}  // namespace

extern "C" ubd_model *ubd_model_load(const ubd_hparams *hparams, const ubd_tensor_src *tensors, int32_t n_tensors,
                                     const ubd_model_params *params, int32_t *status) {
    auto fail = [&](int32_t code, const std::string &msg) -> ubd_model * {
        set_err(msg);
        if (status) *status = code;
        return nullptr;
    };
    g_err.clear();
    const double t0 = now_ms();
    if (!hparams || !tensors || n_tensors <= 0) return fail(-1, "ubd_model_load: missing arguments");
    const ubd_hparams hp = *hparams;
    if (hp.n_layer <= 0 || hp.n_embd <= 0 || hp.n_head <= 0 || hp.n_head_kv <= 0 || hp.n_ff <= 0 || hp.n_vocab <= 0)
        return fail(-1, "ubd_model_load: sizes must be positive");
    if (hp.n_embd % hp.n_head || hp.n_head % hp.n_head_kv) return fail(-1, "ubd_model_load: head counts do not divide");
    const int hd = hp.n_embd / hp.n_head;
    if (hd != 32 && hd != 64 && hd != 128) return fail(-1, "ubd_model_load: head_dim must be 32, 64 or 128");
    if (hp.n_head / hp.n_head_kv > 32) return fail(-1, "ubd_model_load: at most 32 query heads per KV head");
    if (hp.n_embd % 16 || hp.n_ff % 16 || hp.n_vocab % 16)
        return fail(-1, "ubd_model_load: n_embd, n_ff and n_vocab must be multiples of 16");
    if (hp.rope_type != 0) return fail(-1, "ubd_model_load: only rope type 0 is supported");

    const auto expect = expected_tensors(hp);
    std::map<std::string, const ubd_tensor_src *> got;
    int wtype = -1;
    for (int32_t i = 0; i < n_tensors; ++i) {
        const ubd_tensor_src &t = tensors[i];
        if (!t.name || !t.data) return fail(-1, "ubd_model_load: tensor without name or data");
        auto it = expect.find(t.name);
        if (it == expect.end()) return fail(-1, std::string("ubd_model_load: unknown tensor ") + t.name);
        if (got.count(t.name)) return fail(-1, std::string("ubd_model_load: duplicate tensor ") + t.name);
        if (t.ne[0] != it->second.ne0 || t.ne[1] != it->second.ne1)
            return fail(-1, std::string("ubd_model_load: wrong shape for ") + t.name);
        if (it->second.gain) {
            if (t.type != UBD_TYPE_F32) return fail(-1, std::string("ubd_model_load: norm must be F32: ") + t.name);
        } else {
            const int wt = wtype_of(t.type);
            if (wt < 0) return fail(-1, std::string("ubd_model_load: unsupported matrix type for ") + t.name);
            if (wtype >= 0 && wt != wtype) return fail(-1, "ubd_model_load: all matrices must share one type");
            wtype = wt;
            if (t.ne[0] % kstep_of(wt))
                return fail(-1, std::string("ubd_model_load: row length not a multiple of the tile for ") + t.name);
        }
        got[t.name] = &t;
    }
    // The output matrix is optional: without it the model is tied and the
    // logits reuse the token embedding table, which has the same shape
    // {n_embd, n_vocab} ("llama.cpp AI LLM Engine - how it works", Step 6:
    // the output tensor is not required and is then a duplicate of
    // token_embd).
    const bool tied = !got.count("output.weight");
    if (tied && got.count("token_embd.weight")) got["output.weight"] = got["token_embd.weight"];
    for (auto &kv : expect)
        if (!got.count(kv.first)) return fail(-1, "ubd_model_load: missing tensor " + kv.first);
    {
        // the products address each (fused) matrix with 32-bit byte offsets
        const double d = hp.n_embd, kv = (double)hp.n_head_kv * hd, eb = (double)elem_bytes(wtype);
        const double rows_k[][2] = {{d + 2 * kv, d}, {d, d}, {2.0 * hp.n_ff, d}, {d, (double)hp.n_ff},
                                    {(double)hp.n_vocab, d}};
        for (const auto &rk : rows_k)
            if (rk[0] * rk[1] * eb > 2147483647.0)
                return fail(-1, "ubd_model_load: a fused weight matrix exceeds 2 GiB");
    }

    ubd_model *m = new ubd_model();
    m->hp = hp;
    m->head_dim = hd;
    m->wtype = wtype;
    if (params) {
        m->device = params->device;
        m->stream = (hipStream_t)params->stream;
        m->mem.alloc = params->alloc;
        m->mem.free = params->free;
        m->mem.ud = params->alloc_user_data;
    }
    auto bail = [&](int32_t code, const std::string &msg) -> ubd_model * {
        m->mem.release();
        delete m;
        return fail(code, msg);
    };
    if (!hip_ok(hipSetDevice(m->device), "hipSetDevice")) return bail(-2, g_err);
    hipStream_t st = m->stream;

    auto copy_gain = [&](const std::string &name, float **dst) -> bool {
        const ubd_tensor_src &s = *got[name];
        *dst = (float *)m->mem.get((size_t)hp.n_embd * 4);
        if (!*dst) return false;
        return hip_ok(hipMemcpyAsync(*dst, s.data, (size_t)hp.n_embd * 4,
                                     s.on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice, st),
                      "norm upload");
    };
    auto make_mat = [&](DevMat &dm, const std::vector<std::string> &names, int mode) -> bool {
        const ubd_tensor_src &s0 = *got[names[0]];
        const int K = (int)s0.ne[0];
        int rows = 0;
        std::vector<Staged> stg(names.size());
        RelayoutSrc src[3];
        for (size_t i = 0; i < names.size(); ++i) {
            const ubd_tensor_src &s = *got[names[i]];
            if (!stage(s, wtype, st, &stg[i])) return false;
            src[i].data = stg[i].data;
            src[i].scales = stg[i].scales;
            src[i].rows = (int)s.ne[1];
            rows += (int)s.ne[1];
        }
        dm.wtype = wtype;
        dm.rows = rows;
        dm.cols = K;
        dm.w = m->mem.get((size_t)rows * K * elem_bytes(wtype));
        if (!dm.w) return false;
        if (wtype == W_Q8) {
            dm.scales = (uint16_t *)m->mem.get((size_t)rows * (K / 32) * 2);
            if (!dm.scales) return false;
        }
        launch_relayout(wtype, src, (int)names.size(), mode, K, dm.w, dm.scales, st);
        if (!hip_ok(hipGetLastError(), "relayout")) return false;
        // staging buffers are freed when stg goes out of scope: finish first
        return hip_ok(hipStreamSynchronize(st), "relayout sync");
    };

    m->layers.resize(hp.n_layer);
    for (int il = 0; il < hp.n_layer; ++il) {
        const std::string p = "blk." + std::to_string(il) + ".";
        auto &L = m->layers[il];
        if (!copy_gain(p + "attn_norm.weight", &L.attn_norm) || !copy_gain(p + "ffn_norm.weight", &L.ffn_norm))
            return bail(-2, "ubd_model_load: norm upload failed: " + g_err);
        if (!make_mat(L.qkv, {p + "attn_q.weight", p + "attn_k.weight", p + "attn_v.weight"}, 0) ||
            !make_mat(L.o, {p + "attn_output.weight"}, 0) ||
            !make_mat(L.gu, {p + "ffn_gate.weight", p + "ffn_up.weight"}, 1) ||
            !make_mat(L.down, {p + "ffn_down.weight"}, 0))
            return bail(-2, "ubd_model_load: weight upload failed: " + g_err);
    }
    if (!copy_gain("output_norm.weight", &m->out_norm) || !make_mat(m->out, {"output.weight"}, 0))
        return bail(-2, "ubd_model_load: output upload failed: " + g_err);
    {
        const ubd_tensor_src &s = *got["token_embd.weight"];
        const size_t n = (size_t)s.ne[0] * s.ne[1];
        Staged stg;
        if (!stage(s, wtype, st, &stg)) return bail(-2, "ubd_model_load: embedding upload failed: " + g_err);
        m->embd = m->mem.get(n * elem_bytes(wtype));
        if (!m->embd ||
            !hip_ok(hipMemcpyAsync(m->embd, stg.data, n * elem_bytes(wtype), hipMemcpyDeviceToDevice, st), "embedding"))
            return bail(-2, "ubd_model_load: embedding upload failed: " + g_err);
        if (wtype == W_Q8) {
            m->embd_scales = (uint16_t *)m->mem.get(n / 32 * 2);
            if (!m->embd_scales ||
                !hip_ok(hipMemcpyAsync(m->embd_scales, stg.scales, n / 32 * 2, hipMemcpyDeviceToDevice, st), "scales"))
                return bail(-2, "ubd_model_load: embedding upload failed: " + g_err);
        }
        if (!hip_ok(hipStreamSynchronize(st), "embedding sync"))
            return bail(-2, "ubd_model_load: embedding upload failed: " + g_err);
    }
    if (!hip_ok(hipStreamSynchronize(st), "load sync")) return bail(-2, "ubd_model_load: " + g_err);
    m->t_load_ms = now_ms() - t0;
    log_line(1, "model loaded: %d layers, %.1f MiB on device, %.1f ms%s", hp.n_layer, m->mem.bytes / 1048576.0,
             m->t_load_ms, tied ? ", output tied to token_embd" : "");
    if (status) *status = 0;
    return m;
}

extern "C" void ubd_model_free(ubd_model *model) {
    if (!model) return;
    (void)hipSetDevice(model->device);
    (void)hipStreamSynchronize(model->stream);
    model->mem.release();
    delete model;
}

extern "C" size_t ubd_model_size(const ubd_model *model) { return model ? model->mem.bytes : 0; }

// ----------------------------------------------------------------- context
struct ubd_context : public Executor {
    ubd_model *model = nullptr;
    ubd_context_params cp{};
    hipStream_t stream = nullptr;
    Planner planner;
    DevAlloc mem;
    int type_k = KV_F16, type_v = KV_F16;
    size_t kv_layer_elems = 0;              // per layer, K or V
    size_t k_layer_bytes = 0, v_layer_bytes = 0;
    float *kv_stage = nullptr;              // q8_0 caches: [cap][2][Hk*hd] rows awaiting quantisation
    uint32_t cell_stride = 0;               // cells per stream rounded up to 32
    void *k_cache = nullptr, *v_cache = nullptr;
    int32_t *cell_pos = nullptr;            // [stream][cell_stride]
    uint32_t *cell_seq = nullptr;           // [stream][n_seq_words][cell_stride]
    int n_seq_words = 1;
    float *x = nullptr, *q = nullptr;
    Act actA, actB, actC;
    float *part_o = nullptr, *part_ml = nullptr;
    float *split_scratch = nullptr;         // k-slice partial sums of the residual prefill products
                                            // [MAX_K_SLICES][cap][d]
    int max_chunks = 0;                     // f32-path chunks (ATTN_CHUNK cells)
    int max_chunks_mfma = 0;                // MFMA split-path chunks (ATTN_DECODE_CHUNK cells)
    bool mfma_attn = false;
    int attn_wave_slots = 1024;             // split-attention waves resident at once (CUs x SIMDs x waves)
    double *inv_freq = nullptr;
    float2 *rope_cs = nullptr;              // [cap][head_dim / 2] (cos, sin) of the ubatch's angles
    int32_t *info_dev = nullptr;
    int32_t *info_host[2] = {nullptr, nullptr};
    hipEvent_t info_ev[2] = {nullptr, nullptr};
    int info_i = 0;
    int cap = 0;                            // n_ubatch
    float *logits_dev = nullptr;
    int32_t logits_cap = 0;
    std::vector<float> logits_host;
    bool logits_host_valid = false;
    int32_t *argmax_host = nullptr;         // pinned, coherent: the argmax kernel writes the picks here
    bool chain_tok = false;                 // this ubatch's one token id is already in the device table
    std::vector<int32_t> scan_sufmin;       // run_ubatch's per-stream suffix minima of cell positions
    ArgmaxWork argmax_work;
    std::vector<int32_t> last_ub_idx;
    float *dump = nullptr;
    ubd_perf perf{};
    // kernel timing
    uint32_t time_mask = 0;
    std::vector<hipEvent_t> ev_pool;
    struct Pending {
        int cls;
        hipEvent_t a, b;
    };
    std::vector<Pending> pending;
    int32_t t_launches[UBD_KERNEL_CLASSES] = {};
    double t_ms[UBD_KERNEL_CLASSES] = {};

    hipEvent_t take_event() {
        if (!ev_pool.empty()) {
            hipEvent_t e = ev_pool.back();
            ev_pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        (void)hipEventCreate(&e);
        return e;
    }
    template <typename F>
    void timed(int cls, F &&launch) {
        if (!(time_mask & (1u << cls))) {
            launch();
            return;
        }
        hipEvent_t a = take_event(), b = take_event();
        g_launch_timing = {a, b};
        launch();
        g_launch_timing = {};
        pending.push_back({cls, a, b});
    }
    void collect_timing() {
        (void)hipStreamSynchronize(stream);
        for (auto &p : pending) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
                t_ms[p.cls] += ms;
                t_launches[p.cls] += 1;
            }
            ev_pool.push_back(p.a);
            ev_pool.push_back(p.b);
        }
        pending.clear();
    }

    // The token table of a ubatch of T tokens: sections of T ints (tiles: 4
    // per tile, at most T tiles), so a one-token step uploads a few dozen
    // bytes; its addresses depend on T alone, which a step's graph fixes.
    TokInfo tok_info(int T) const {
        TokInfo t;
        const int32_t *b = info_dev;
        t.token = b;
        t.pos = b + T;
        t.seq = b + 2 * T;
        t.stream = b + 3 * T;
        t.cell = b + 4 * T;
        t.out_row = b + 5 * T;
        t.tile_of = b + 6 * T;
        t.out_tok = b + 7 * T;
        t.tiles = b + 9 * T;
        t.seqw = (const uint32_t *)(b + 13 * T);
        t.n_seq_words = n_seq_words;
        return t;
    }
    const int32_t *out_lrow(int T) const { return info_dev + 8 * T; }
    size_t info_ints(int T) const { return (size_t)(13 + n_seq_words) * T; }

    // ---- decode-step graphs: each ubatch shape is captured once on
    // cap_stream and replayed on the context stream from then on.  Every kernel of
    // the step reads the per-ubatch values (tokens, positions, cells, tiles,
    // scan lengths) from the token table, so a shape's graph stays valid
    // from step to step; what its launches take by value is in the key.
    struct GraphKey {
        int T, n_out, n_tiles, chunk_cells, n_chunks;
        bool operator<(const GraphKey &o) const {
            if (T != o.T) return T < o.T;
            if (n_out != o.n_out) return n_out < o.n_out;
            if (n_tiles != o.n_tiles) return n_tiles < o.n_tiles;
            if (chunk_cells != o.chunk_cells) return chunk_cells < o.chunk_cells;
            return n_chunks < o.n_chunks;
        }
    };
    struct GraphSlot {
        hipGraphExec_t exec = nullptr;
        uint64_t last_use = 0;
    };
    static constexpr size_t kGraphSlots = 16;
    std::map<GraphKey, GraphSlot> graphs;
    uint64_t graph_clock = 0;
    uint32_t graph_gen = 0;
    hipStream_t cap_stream = nullptr;
    bool graphs_on = true;
    void clear_graphs() {
        if (graphs.empty()) return;
        (void)hipStreamSynchronize(stream);
        for (auto &kv : graphs) (void)hipGraphExecDestroy(kv.second.exec);
        graphs.clear();
    }
    int32_t forward_graph(const GraphKey &key);
    int32_t enqueue_forward(hipStream_t s, const GraphKey &key);

    int32_t reserve_outputs(int32_t n) override;
    int32_t run_ubatch(const UBatch &ub, int32_t k) override;
    int32_t cells_changed(const std::vector<uint8_t> &touched) override;
    int32_t stream_copy(int32_t src, int32_t dst) override;
    int32_t cells_move(const std::vector<std::vector<int32_t>> &src) override;
    bool sync_cell_tables(int32_t stream);
};

extern "C" ubd_context_params ubd_context_default_params(void) {
    ubd_context_params p{};
    p.n_ctx = 0;
    p.n_batch = 2048;
    p.n_ubatch = 512;
    p.n_seq_max = 1;
    p.type_k = UBD_TYPE_F16;
    p.type_v = UBD_TYPE_F16;
    p.kv_unified = false;
    p.graph_reuse = true;
    return p;
}

extern "C" ubd_context *ubd_init_from_model(ubd_model *model, const ubd_context_params *params, int32_t *status) {
    g_err.clear();
    auto fail = [&](int32_t code, const std::string &msg) -> ubd_context * {
        set_err(msg);
        if (status) *status = code;
        return nullptr;
    };
    if (!model || !params) return fail(-1, "ubd_init_from_model: missing arguments");
    const ubd_context_params cp = *params;
    auto kvt = [](ubd_type t) {
        return t == UBD_TYPE_F32 ? KV_F32 : t == UBD_TYPE_F16 ? KV_F16 : t == UBD_TYPE_Q8_0 ? KV_Q8 : -1;
    };
    if (kvt(cp.type_k) < 0 || kvt(cp.type_v) < 0)
        return fail(-1, "ubd_init_from_model: KV types must be F32, F16 or Q8_0");
    if ((kvt(cp.type_k) == KV_Q8) != (kvt(cp.type_v) == KV_Q8))
        return fail(-1, "ubd_init_from_model: a Q8_0 KV cache needs type_k == type_v == Q8_0");
    if (kvt(cp.type_k) == KV_Q8 && !attn_mfma_ok(KV_Q8, KV_Q8, model->head_dim, model->hp.n_head / model->hp.n_head_kv))
        return fail(-1, "ubd_init_from_model: a Q8_0 KV cache needs head_dim 32, 64 or 128 and n_head / n_head_kv <= 16");
    ubd_context *c = new ubd_context();
    c->model = model;
    c->cp = cp;
    c->stream = (hipStream_t)cp.stream;
    c->graphs_on = cp.graph_reuse;
    c->type_k = kvt(cp.type_k);
    c->type_v = kvt(cp.type_v);
    c->mem.alloc = model->mem.alloc;
    c->mem.free = model->mem.free;
    c->mem.ud = model->mem.ud;
    std::string err;
    const ubd_hparams &hp = model->hp;
    if (c->planner.init(cp.n_ctx ? cp.n_ctx : (uint32_t)hp.n_ctx_train, cp.n_batch, cp.n_ubatch, cp.n_seq_max,
                        cp.kv_unified, hp.n_vocab, &err) != UBD_OK) {
        delete c;
        return fail(-1, "ubd_init_from_model: " + err);
    }
    auto bail = [&](const std::string &msg) -> ubd_context * {
        c->mem.release();
        for (int i = 0; i < 2; ++i) {
            if (c->info_host[i]) (void)hipHostFree(c->info_host[i]);
            if (c->info_ev[i]) (void)hipEventDestroy(c->info_ev[i]);
        }
        if (c->argmax_host) (void)hipHostFree(c->argmax_host);
        delete c;
        return fail(-2, "ubd_init_from_model: " + msg + (g_err.empty() ? "" : ": " + g_err));
    };
    if (!hip_ok(hipSetDevice(model->device), "hipSetDevice")) return bail("device");
    const Planner &P = c->planner;
    const int hd = model->head_dim, H = hp.n_head, Hk = hp.n_head_kv, d = hp.n_embd, F = hp.n_ff;
    c->cap = (int)P.n_ubatch;
    c->cell_stride = (P.n_cells + 31) / 32 * 32;
    const size_t cells = (size_t)P.n_stream * c->cell_stride;
    c->kv_layer_elems = cells * Hk * hd;
    c->k_layer_bytes = kv_layer_bytes(c->type_k, c->kv_layer_elems);
    c->v_layer_bytes = kv_layer_bytes(c->type_v, c->kv_layer_elems);
    c->k_cache = c->mem.get(c->k_layer_bytes * hp.n_layer);
    c->v_cache = c->mem.get(c->v_layer_bytes * hp.n_layer);
    c->n_seq_words = P.cells.n_seq_words();
    c->cell_pos = (int32_t *)c->mem.get(cells * 4);
    c->cell_seq = (uint32_t *)c->mem.get(cells * c->n_seq_words * 4);
    if (!c->k_cache || !c->v_cache || !c->cell_pos || !c->cell_seq) return bail("KV cache allocation failed");
    // zero K/V: masked cells still enter P*V with weight 0, so never-written
    // cells must hold finite values
    if (!hip_ok(hipMemsetAsync(c->k_cache, 0, c->k_layer_bytes * hp.n_layer, c->stream), "memset") ||
        !hip_ok(hipMemsetAsync(c->v_cache, 0, c->v_layer_bytes * hp.n_layer, c->stream), "memset"))
        return bail("KV cache init failed");
    if (!hip_ok(hipMemsetAsync(c->cell_pos, 0xff, cells * 4, c->stream), "memset") ||
        !hip_ok(hipMemsetAsync(c->cell_seq, 0, cells * c->n_seq_words * 4, c->stream), "memset"))
        return bail("KV cell table init failed");
    const int cap = c->cap;
    const bool f32w = model->wtype == W_F32;
    // (HILO planes hold whole 16-token tiles: the prefill products read them tiled)
    auto make_act = [&](Act &a, int ld) -> bool {
        a.ld = ld;
        if (f32w) {
            a.f32 = (float *)c->mem.get((size_t)cap * ld * 4);
            return a.f32 != nullptr;
        }
        const size_t rows = ((size_t)cap + 15) / 16 * 16;
        a.hi = (uint16_t *)c->mem.get(rows * ld * 2);
        a.lo = (uint16_t *)c->mem.get(rows * ld * 2);
        return a.hi && a.lo;
    };
    c->x = (float *)c->mem.get((size_t)cap * d * 4);
    c->q = (float *)c->mem.get((size_t)cap * H * hd * 4);
    if (c->type_k == KV_Q8) {
        c->kv_stage = (float *)c->mem.get((size_t)cap * 2 * Hk * hd * 4);
        if (!c->kv_stage) return bail("KV staging allocation failed");
    }
    if (!c->x || !c->q || !make_act(c->actA, d) || !make_act(c->actB, H * hd) || !make_act(c->actC, F))
        return bail("activation allocation failed");
    c->max_chunks = (int)((P.n_cells + ATTN_CHUNK - 1) / ATTN_CHUNK);
    c->max_chunks_mfma = (int)((P.n_cells + ATTN_DECODE_CHUNK - 1) / ATTN_DECODE_CHUNK);
    c->mfma_attn = attn_mfma_ok(c->type_k, c->type_v, hd, H / Hk);
    {
        // waves of the split attention kernel per SIMD (its registers:
        // head size 128 fits one, 64 two, 32 four), 4 SIMDs per CU
        int n_cu = 0;
        if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, model->device) != hipSuccess ||
            n_cu <= 0)
            n_cu = 256;
        c->attn_wave_slots = n_cu * 4 * (hd >= 128 ? 1 : hd >= 64 ? 2 : 4);
    }
    // split partials: f32 path up to n_ubatch tokens; MFMA path only for <= 16 tokens
    const size_t part_rows = c->mfma_attn ? (size_t)std::min(cap, 16) * H * c->max_chunks_mfma
                                          : (size_t)cap * H * c->max_chunks;
    c->part_o = (float *)c->mem.get(part_rows * hd * 4);
    c->part_ml = (float *)c->mem.get(part_rows * 2 * 4);

    if (!c->part_o || !c->part_ml) return bail("attention scratch allocation failed");
    if ((model->wtype == W_BF16 || model->wtype == W_Q8) && cap >= 64) {
        c->split_scratch = (float *)c->mem.get((size_t)MAX_K_SLICES * cap * d * 4);
        if (!c->split_scratch) return bail("product scratch allocation failed");
    }
    std::vector<double> inv(hd / 2);
    for (int i = 0; i < hd / 2; ++i) inv[i] = std::pow((double)hp.rope_freq_base, -2.0 * i / hd);
    c->inv_freq = (double *)c->mem.get(inv.size() * sizeof(double));
    c->rope_cs = (float2 *)c->mem.get((size_t)cap * (hd / 2) * sizeof(float2));
    c->info_dev = (int32_t *)c->mem.get(c->info_ints(c->cap) * 4);
    const size_t amax_rows = std::max<uint32_t>(P.n_batch, 1);
    c->argmax_work.pv = (float *)c->mem.get(amax_rows * ARGMAX_BLOCKS * 4);
    c->argmax_work.pi = (int32_t *)c->mem.get(amax_rows * ARGMAX_BLOCKS * 4);
    c->argmax_work.counter = (int32_t *)c->mem.get(amax_rows * 4);
    if (!c->inv_freq || !c->rope_cs || !c->info_dev || !c->argmax_work.pv || !c->argmax_work.pi ||
        !c->argmax_work.counter)
        return bail("allocation failed");
    if (!hip_ok(hipMemsetAsync(c->argmax_work.counter, 0, amax_rows * 4, c->stream), "memset"))
        return bail("counter init failed");
    if (!hip_ok(hipMemcpyAsync(c->inv_freq, inv.data(), inv.size() * sizeof(double), hipMemcpyHostToDevice,
                               c->stream), "upload"))
        return bail("upload failed");
    for (int i = 0; i < 2; ++i) {
        if (!hip_ok(hipHostMalloc((void **)&c->info_host[i], c->info_ints(c->cap) * 4, hipHostMallocDefault), "pinned") ||
            !hip_ok(hipEventCreateWithFlags(&c->info_ev[i], hipEventDisableTiming), "event"))
            return bail("pinned staging allocation failed");
    }
    if (!hip_ok(hipHostMalloc((void **)&c->argmax_host,
                              (size_t)std::max<uint32_t>(P.n_batch, UBD_GREEDY_CHAIN_BLOCK) * 4,
                              hipHostMallocCoherent), "pinned"))
        return bail("pinned argmax buffer allocation failed");
    if (!hip_ok(hipStreamSynchronize(c->stream), "init sync")) return bail("sync failed");
    log_line(1, "context: n_ctx %u (%u streams x %u cells), n_batch %u, n_ubatch %u, KV %.1f MiB", P.n_ctx,
             P.n_stream, P.n_cells, P.n_batch, P.n_ubatch,
             (double)(c->k_layer_bytes + c->v_layer_bytes) * hp.n_layer / 1048576.0);
    if (status) *status = 0;
    return c;
}

extern "C" void ubd_free(ubd_context *ctx) {
    if (!ctx) return;
    (void)hipSetDevice(ctx->model->device);
    (void)hipStreamSynchronize(ctx->stream);
    ctx->collect_timing();
    ctx->clear_graphs();
    if (ctx->cap_stream) (void)hipStreamDestroy(ctx->cap_stream);
    for (hipEvent_t e : ctx->ev_pool) (void)hipEventDestroy(e);
    ctx->mem.release();
    for (int i = 0; i < 2; ++i) {
        if (ctx->info_host[i]) (void)hipHostFree(ctx->info_host[i]);
        if (ctx->info_ev[i]) (void)hipEventDestroy(ctx->info_ev[i]);
    }
    if (ctx->argmax_host) (void)hipHostFree(ctx->argmax_host);
    delete ctx;
}

extern "C" uint32_t ubd_n_ctx(const ubd_context *ctx) { return ctx ? ctx->planner.n_ctx : 0; }
extern "C" uint32_t ubd_n_batch(const ubd_context *ctx) { return ctx ? ctx->planner.n_batch : 0; }
extern "C" uint32_t ubd_n_ubatch(const ubd_context *ctx) { return ctx ? ctx->planner.n_ubatch : 0; }

int32_t ubd_context::reserve_outputs(int32_t n) {
    logits_host_valid = false;
    if (n <= logits_cap) return UBD_OK;
    const ubd_hparams &hp = model->hp;
    int32_t want = std::max<int32_t>(n, 1);
    // logits rows live as long as the context; an outgrown block is kept
    float *p = (float *)mem.get((size_t)want * hp.n_vocab * 4);
    if (!p) {
        set_err("cannot allocate the logits buffer");
        return UBD_ALLOC_FAILED;
    }
    clear_graphs();
    logits_dev = p;
    logits_cap = want;
    return UBD_OK;
}

bool ubd_context::sync_cell_tables(int32_t st) {
    const Planner &P = planner;
    bool ok = hip_ok(hipMemcpyAsync(cell_pos + (size_t)st * cell_stride, P.cells.pos_data(st),
                                    (size_t)P.n_cells * 4, hipMemcpyHostToDevice, stream),
                     "cell table upload");
    for (int w = 0; ok && w < n_seq_words; ++w)
        ok = hip_ok(hipMemcpyAsync(cell_seq + ((size_t)st * n_seq_words + w) * cell_stride,
                                   P.cells.seq_words(st) + (size_t)w * P.n_cells, (size_t)P.n_cells * 4,
                                   hipMemcpyHostToDevice, stream),
                    "cell table upload");
    return ok && hip_ok(hipStreamSynchronize(stream), "cell table sync");
}

int32_t ubd_context::cells_changed(const std::vector<uint8_t> &touched) {
    for (uint32_t st = 0; st < planner.n_stream; ++st)
        if (touched[st] && !sync_cell_tables((int32_t)st)) return UBD_COMPUTE_FAILED;
    return UBD_OK;
}

int32_t ubd_context::stream_copy(int32_t src, int32_t dst) {
    const ubd_hparams &hp = model->hp;
    const size_t per_stream = kv_layer_elems / planner.n_stream;     // values of one stream in one layer
    auto copy = [&](void *base, size_t layer_bytes, int type) -> bool {
        const size_t esz = type == KV_F32 ? 4 : type == KV_F16 ? 2 : 1;
        for (int il = 0; il < hp.n_layer; ++il) {
            char *l = (char *)base + layer_bytes * il;
            if (!hip_ok(hipMemcpyAsync(l + dst * per_stream * esz, l + src * per_stream * esz, per_stream * esz,
                                       hipMemcpyDeviceToDevice, stream),
                        "stream copy"))
                return false;
            if (type == KV_Q8) {
                char *sc = l + kv_layer_elems;
                const size_t sb = per_stream / 32 * 2;
                if (!hip_ok(hipMemcpyAsync(sc + dst * sb, sc + src * sb, sb, hipMemcpyDeviceToDevice, stream),
                            "stream copy"))
                    return false;
            }
        }
        return true;
    };
    (void)hipSetDevice(model->device);
    if (!copy(k_cache, k_layer_bytes, type_k) || !copy(v_cache, v_layer_bytes, type_v) ||
        !hip_ok(hipStreamSynchronize(stream), "stream copy sync"))
        return UBD_COMPUTE_FAILED;
    return UBD_OK;
}

int32_t ubd_context::cells_move(const std::vector<std::vector<int32_t>> &src) {
    const ubd_hparams &hp = model->hp;
    const int hd = model->head_dim, Hk = hp.n_head_kv;
    (void)hipSetDevice(model->device);
    int32_t rc = UBD_OK;
    for (uint32_t st = 0; st < planner.n_stream && rc == UBD_OK; ++st) {
        // only the cells whose index changes
        std::vector<int32_t> from, to;
        for (size_t j = 0; j < src[st].size(); ++j)
            if (src[st][j] != (int32_t)j) {
                from.push_back(src[st][j]);
                to.push_back((int32_t)j);
            }
        const int n = (int)from.size();
        if (n == 0) continue;
        int32_t *dcells = nullptr;
        void *tmp = nullptr;
        const size_t tb = std::max(kv_move_tmp_bytes(type_k, n, Hk, hd), kv_move_tmp_bytes(type_v, n, Hk, hd));
        bool ok = hip_ok(hipMalloc(&dcells, (size_t)2 * n * 4), "defrag alloc") &&
                  hip_ok(hipMalloc(&tmp, tb), "defrag alloc") &&
                  hip_ok(hipMemcpy(dcells, from.data(), (size_t)n * 4, hipMemcpyHostToDevice), "defrag cells") &&
                  hip_ok(hipMemcpy(dcells + n, to.data(), (size_t)n * 4, hipMemcpyHostToDevice), "defrag cells");
        for (int il = 0; ok && il < hp.n_layer; ++il)
            for (int which = 0; which < 2; ++which) {
                void *cache = which == 0 ? (char *)k_cache + k_layer_bytes * il : (char *)v_cache + v_layer_bytes * il;
                const int type = which == 0 ? type_k : type_v;
                // every source row is in tmp before any destination is written
                launch_kv_move(cache, type, which == 1, (int)st, dcells, n, Hk, hd, (int)cell_stride,
                               kv_layer_elems, tmp, true, stream);
                launch_kv_move(cache, type, which == 1, (int)st, dcells + n, n, Hk, hd, (int)cell_stride,
                               kv_layer_elems, tmp, false, stream);
            }
        ok = ok && hip_ok(hipGetLastError(), "kv_move") && hip_ok(hipStreamSynchronize(stream), "defrag sync");
        if (dcells) (void)hipFree(dcells);
        if (tmp) (void)hipFree(tmp);
        if (!ok) rc = UBD_COMPUTE_FAILED;
    }
    return rc;
}

int32_t ubd_context::run_ubatch(const UBatch &ub, int32_t k) {
    (void)k;
    if (cp.abort_callback && cp.abort_callback(cp.abort_user_data)) {
        set_err("decode aborted by the callback");
        return UBD_ABORTED;
    }
    const ubd_model &M = *model;
    const ubd_hparams &hp = M.hp;
    const int T = ub.size();
    const int hd = M.head_dim, H = hp.n_head, Hk = hp.n_head_kv;
    const int G = H / Hk;

    // ---- per-ubatch token table (one H2D copy from pinned staging)
    const int bi = info_i;
    info_i ^= 1;
    if (!hip_ok(hipEventSynchronize(info_ev[bi]), "staging reuse")) return UBD_COMPUTE_FAILED;
    int32_t *h = info_host[bi];
    std::fill(h, h + info_ints(T), 0);
    int n_out = 0;
    for (int t = 0; t < T; ++t) {
        h[t] = ub.token[t];
        h[T + t] = ub.pos[t];
        h[2 * T + t] = ub.seq[t];
        h[3 * T + t] = ub.stream[t];
        h[4 * T + t] = ub.cell[t];
        h[5 * T + t] = ub.out_row[t];
        for (int w = 0; w < n_seq_words; ++w) h[13 * T + t * n_seq_words + w] = (int32_t)ub.seqw[(size_t)t * n_seq_words + w];
        if (ub.out_row[t] >= 0) {
            h[7 * T + n_out] = t;
            h[8 * T + n_out] = ub.out_row[t];
            ++n_out;
        }
    }
    const bool split = T <= 16;
    int max_scan = 0;
    const int qt = mfma_attn ? std::max(1, 16 / G) : std::max(1, attn_tile_rows(hd) / G);
    int n_tiles = 0;
    // per stream, the smallest position in cells [c, n_kv): no cell past the
    // last c whose suffix holds a position <= P is visible to a token at P
    int sufmin_st = -1;
    std::vector<int32_t> &sufmin = scan_sufmin;
    for (int t = 0; t < T;) {
        int e = t + 1;
        while (e < T && e - t < qt && ub.stream[e] == ub.stream[t]) ++e;
        int32_t *tl = h + 9 * T + 4 * n_tiles;
        tl[0] = t;
        tl[1] = e - t;
        tl[2] = ub.stream[t];
        tl[3] = planner.cells.n_kv(ub.stream[t]);
        if (mfma_attn && !split && tl[3] <= 8192) {
            // scan only up to the last cell some token of the tile can see
            const int st = ub.stream[t];
            const int nkv = tl[3];
            if (sufmin_st != st) {
                sufmin.assign((size_t)nkv + 1, INT32_MAX);
                for (int c = nkv - 1; c >= 0; --c) {
                    const int32_t p = planner.cells.pos_at(st, c);
                    sufmin[c] = std::min(p < 0 ? INT32_MAX : p, sufmin[c + 1]);
                }
                sufmin_st = st;
            }
            int32_t pmax = ub.pos[t];
            for (int j = t + 1; j < e; ++j) pmax = std::max(pmax, ub.pos[j]);
            // the exact scan starts at the last cell whose position is <= pmax
            // (the first c with sufmin[c] > pmax, less one: sufmin rises with c)
            int c = (int)(std::upper_bound(sufmin.begin(), sufmin.begin() + nkv, pmax) - sufmin.begin()) - 1;
            for (; c >= 0; --c) {
                const int cpp = planner.cells.pos_at(st, c);
                bool vis = false;
                for (int j = t; j < e && !vis; ++j)
                    vis = cpp >= 0 && cpp <= ub.pos[j] && planner.cells.has(st, c, ub.seq[j]);
                if (vis) break;
            }
            tl[3] = c + 1;
        }
        for (int j = t; j < e; ++j) h[6 * T + j] = n_tiles;
        max_scan = std::max(max_scan, (int)tl[3]);
        ++n_tiles;
        t = e;
    }
    // (a chained greedy step's token id was written into the table by the
    // previous step's argmax: the upload leaves that word alone)
    const int skip = chain_tok && T == 1 ? 1 : 0;
    if (!hip_ok(hipMemcpyAsync(info_dev + skip, h + skip, (info_ints(T) - skip) * 4, hipMemcpyHostToDevice, stream),
                "token table upload") ||
        !hip_ok(hipEventRecord(info_ev[bi], stream), "event"))
        return UBD_COMPUTE_FAILED;
    last_ub_idx = ub.idx;

    // split-attention chunk geometry (MFMA path, ubatches of <= 16 tokens):
    // from the scan length rounded up to a multiple of 256 cells, so
    // consecutive decode steps launch the same grid (the kernels read each
    // tile's exact scan length from the token table; chunks past it are
    // empty).  One round of waves: as many chunks as the GPU holds
    // split-kernel waves at once (a second, partial round cost config 4
    // ~7 %), shared by the (tile, KV head) pairs; at least 64 cells each
    // (short scans: 32-cell chunks cost config 3 decode ~3 %).
    GraphKey key{T, n_out, n_tiles, 0, 0};
    if (mfma_attn && split) {
        const int scan = std::min((max_scan + 255) / 256 * 256, (int)cell_stride);
        const int pairs = std::max(1, n_tiles * Hk);
        const int per_pair = std::max(1, attn_wave_slots / pairs);
        const int want = (scan + per_pair - 1) / per_pair;
        const int cmin = std::max(ATTN_DECODE_CHUNK, g_tuning.attn_chunk_min / 32 * 32);
        key.chunk_cells = std::max(cmin, (want + 31) / 32 * 32);
        key.n_chunks = std::max(1, (scan + key.chunk_cells - 1) / key.chunk_cells);
    }
    const bool graph = graphs_on && time_mask == 0 && !dump;
    const int32_t rc = graph ? forward_graph(key) : enqueue_forward(stream, key);
    if (rc == UBD_OK) perf.n_ubatch += 1;
    return rc;
}

int32_t ubd_context::forward_graph(const GraphKey &key) {
    if (graph_gen != g_tuning_gen) {
        clear_graphs();
        graph_gen = g_tuning_gen;
    }
    auto it = graphs.find(key);
    if (it != graphs.end()) {
        it->second.last_use = ++graph_clock;
        perf.n_reused += 1;
        return hip_ok(hipGraphLaunch(it->second.exec, stream), "graph launch") ? UBD_OK : UBD_COMPUTE_FAILED;
    }
    // a new shape: record its kernels on the capture stream (nothing runs
    // there), then launch the graph on the context stream
    if (!cap_stream && hipStreamCreateWithFlags(&cap_stream, hipStreamNonBlocking) != hipSuccess) {
        (void)hipGetLastError();
        cap_stream = nullptr;
        graphs_on = false;
        log_line(1, "decode graphs off: no capture stream");
        return enqueue_forward(stream, key);
    }
    if (hipStreamBeginCapture(cap_stream, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        (void)hipGetLastError();
        graphs_on = false;
        log_line(1, "decode graphs off: stream capture unavailable");
        return enqueue_forward(stream, key);
    }
    const int32_t rc = enqueue_forward(cap_stream, key);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(cap_stream, &g);
    hipGraphExec_t exec = nullptr;
    const bool ok = rc == UBD_OK && e == hipSuccess && g && hipGraphInstantiateWithFlags(&exec, g, 0) == hipSuccess;
    if (g) (void)hipGraphDestroy(g);
    if (rc != UBD_OK) return rc;     // a refused product: the eager path's error
    if (!ok) {
        (void)hipGetLastError();
        graphs_on = false;
        log_line(1, "decode graphs off: capture or instantiation failed");
        return enqueue_forward(stream, key);
    }
    if (graphs.size() >= kGraphSlots) {
        auto lru = graphs.begin();
        for (auto j = graphs.begin(); j != graphs.end(); ++j)
            if (j->second.last_use < lru->second.last_use) lru = j;
        (void)hipStreamSynchronize(stream);
        (void)hipGraphExecDestroy(lru->second.exec);
        graphs.erase(lru);
    }
    GraphSlot &slot = graphs[key];
    slot.exec = exec;
    slot.last_use = ++graph_clock;
    perf.n_graphs += 1;
    return hip_ok(hipGraphLaunch(exec, stream), "graph launch") ? UBD_OK : UBD_COMPUTE_FAILED;
}

// Every kernel of one ubatch's forward pass, enqueued on s (the context
// stream, or the capture stream while a graph is recorded).
int32_t ubd_context::enqueue_forward(hipStream_t s, const GraphKey &key) {
    const ubd_model &M = *model;
    const ubd_hparams &hp = M.hp;
    const int T = key.T, n_out = key.n_out, n_tiles = key.n_tiles;
    const int hd = M.head_dim, H = hp.n_head, Hk = hp.n_head_kv, d = hp.n_embd;
    const bool split = T <= 16;
    const TokInfo ti = tok_info(T);
    const int n_cells = (int)cell_stride;   // per-s stride of the device KV and cell tables
    const int ph = T > 16 ? 1 : 0;
    bool launched = true;     // every product accepted its arguments
    timed(0 + ph, [&] { launch_embed(M.wtype, M.embd, M.embd_scales, d, ti, T, x, cell_pos, cell_seq, n_cells, inv_freq,
                                       hd / 2, rope_cs, s); });
    if (dump) hip_ok(hipMemcpyAsync(dump, x, (size_t)T * d * 4, hipMemcpyDeviceToDevice, s), "dump");

    // set when the previous layer's down product ran this layer's attention
    // norm in its k-slice pass (LinearArgs::post)
    bool attn_normed = false;
    for (int il = 0; il < hp.n_layer; ++il) {
        const auto &L = M.layers[il];
        const bool fuse_norm = g_tuning.fuse_norm != 0 && linear_norm_fits(T, d);
        const bool fuse_norm_ffn = fuse_norm && g_tuning.fuse_norm == 1;
        LinearArgs la;
        la.wtype = M.wtype;
        la.T = T;
        la.tok = ti;
        // Q, K, V (+RoPE, +append into the KV cells)
        la.w = L.qkv.w;
        la.wscale = L.qkv.scales;
        la.N = L.qkv.rows;
        la.K = L.qkv.cols;
        la.x = actA;
        la.epi = EPI_QKV;
        la.prod = PROD_QKV;
        la.qkv.n_q_rows = H * hd;
        la.qkv.n_k_rows = Hk * hd;
        la.qkv.head_dim = hd;
        la.qkv.n_head_kv = Hk;
        la.qkv.n_cells = n_cells;
        la.qkv.rope_cs = rope_cs;
        la.qkv.q_out = q;
        la.qkv.k_cache = (char *)k_cache + k_layer_bytes * il;
        la.qkv.v_cache = (char *)v_cache + v_layer_bytes * il;
        la.qkv.kv_stage = kv_stage;
        la.qkv.type_k = type_k;
        la.qkv.type_v = type_v;
        if (fuse_norm) la.norm = NormIn{x, nullptr, L.attn_norm, hp.rms_eps, d};
        // the products that read tiled activations get them from their producer tiled
        la.x.tiled = linear_reads_tiled(la);
        if (!fuse_norm && !attn_normed)
            timed(2 + ph, [&] { launch_rmsnorm(x, d, nullptr, T, L.attn_norm, d, hp.rms_eps, la.x, s); });
        attn_normed = false;
        timed(4 + ph, [&] {
            launched &= launch_linear(la, s);
            if (type_k == KV_Q8) {
                // the epilogue staged the f32 K / V rows: quantise them into their cells
                const int ne = Hk * hd;
                launch_kv_quant(kv_stage, KV_F32, 2 * ne, T, ti.cell, ti.stream, 0, la.qkv.k_cache, false, Hk, hd,
                                n_cells, kv_layer_elems, s);
                launch_kv_quant(kv_stage + ne, KV_F32, 2 * ne, T, ti.cell, ti.stream, 0, la.qkv.v_cache, true, Hk, hd,
                                n_cells, kv_layer_elems, s);
            }
        });

        AttnArgs aa;
        aa.q = q;
        aa.k_cache = la.qkv.k_cache;
        aa.v_cache = la.qkv.v_cache;
        aa.type_k = type_k;
        aa.type_v = type_v;
        aa.layer_elems = kv_layer_elems;
        aa.cell_pos = cell_pos;
        aa.cell_seq = cell_seq;
        aa.n_seq_words = n_seq_words;
        aa.n_cells = n_cells;
        aa.n_head = H;
        aa.n_head_kv = Hk;
        aa.head_dim = hd;
        aa.tok = ti;
        aa.T = T;
        aa.n_tiles = n_tiles;
        aa.part_o = part_o;
        aa.part_ml = part_ml;
        LinearArgs lo;
        lo.wtype = M.wtype;
        lo.T = T;
        lo.tok = ti;
        lo.w = L.o.w;
        lo.wscale = L.o.scales;
        lo.N = L.o.rows;
        lo.K = L.o.cols;
        lo.x = actB;
        lo.epi = EPI_RESID;
        lo.prod = PROD_O;
        lo.y = x;
        lo.ldy = d;
        lo.split_out = split_scratch;
        lo.x.tiled = linear_reads_tiled(lo);
        aa.out = lo.x;
        if (mfma_attn) {
            aa.split = split;
            aa.waves = g_tuning.attn_pair ? 2 : 1;
            // split scans that stream at least attn_nt_mb MB of K/V per launch
            // (read once, far past any cache) load it non-temporally: at 16 x
            // 32 K cells 316 against 371 us per layer; short scans and the
            // prefill tiles, which re-read K/V, keep the cached loads
            const double kv_mb = (double)n_tiles * Hk * key.chunk_cells * key.n_chunks * hd * 2 *
                                 (type_k == KV_Q8 ? 1.0625 : 2.0) / 1048576.0;
            aa.kv_nt = split && g_tuning.attn_nt_mb >= 0 && kv_mb >= g_tuning.attn_nt_mb;
            aa.max_chunks = max_chunks_mfma;
            aa.chunk_cells = key.chunk_cells;
            aa.n_chunks_launch = key.n_chunks;
            timed(6 + ph, [&] { launch_attention_mfma(aa, s); });
        } else {
            aa.max_chunks = max_chunks;
            timed(6 + ph, [&] { launch_attention(aa, s); });
        }

        LinearArgs lg = lo;
        lg.w = L.gu.w;
        lg.wscale = L.gu.scales;
        lg.N = L.gu.rows;
        lg.K = L.gu.cols;
        lg.x = actA;
        lg.epi = EPI_SWIGLU;
        lg.prod = PROD_GATE_UP;
        if (fuse_norm_ffn) lg.norm = NormIn{x, nullptr, L.ffn_norm, hp.rms_eps, d};
        lg.x.tiled = linear_reads_tiled(lg);
        // the FFN norm: in the O product's k-slice pass when it splits k
        bool ffn_normed = false;
        if (!fuse_norm_ffn) {
            lo.post = NormOut{L.ffn_norm, hp.rms_eps, lg.x};
            lo.post_done = &ffn_normed;
        }
        timed(8 + ph, [&] { launched &= launch_linear(lo, s); });
        if (!fuse_norm_ffn && !ffn_normed)
            timed(2 + ph, [&] { launch_rmsnorm(x, d, nullptr, T, L.ffn_norm, d, hp.rms_eps, lg.x, s); });
        LinearArgs ld = lo;
        ld.norm = NormIn{};
        ld.post = NormOut{};
        ld.post_done = nullptr;
        if (il + 1 < hp.n_layer && !fuse_norm) {
            ld.post = NormOut{M.layers[il + 1].attn_norm, hp.rms_eps, la.x};
            ld.post_done = &attn_normed;
        }
        ld.w = L.down.w;
        ld.prod = PROD_DOWN;
        ld.wscale = L.down.scales;
        ld.N = L.down.rows;
        ld.K = L.down.cols;
        ld.x = actC;
        ld.x.tiled = linear_reads_tiled(ld);
        lg.out = ld.x;
        timed(10 + ph, [&] { launched &= launch_linear(lg, s); });
        timed(12 + ph, [&] { launched &= launch_linear(ld, s); });
        if (dump)
            hip_ok(hipMemcpyAsync(dump + (size_t)(il + 1) * cap * d, x, (size_t)T * d * 4, hipMemcpyDeviceToDevice,
                                  s), "dump");
    }
    if (n_out > 0) {
        const bool fuse_norm = g_tuning.fuse_norm == 1 && linear_norm_fits(n_out, d);
        LinearArgs lz;
        lz.wtype = M.wtype;
        lz.w = M.out.w;
        lz.wscale = M.out.scales;
        lz.N = M.out.rows;
        lz.K = M.out.cols;
        lz.x = actA;
        lz.T = n_out;
        lz.epi = EPI_LOGITS;
        lz.prod = PROD_LOGITS;
        lz.row_map = out_lrow(T);
        lz.logits = logits_dev;
        if (fuse_norm) lz.norm = NormIn{x, ti.out_tok, M.out_norm, hp.rms_eps, d};
        lz.x.tiled = linear_reads_tiled(lz);
        if (!fuse_norm)
            timed(2 + ph, [&] { launch_rmsnorm(x, d, ti.out_tok, n_out, M.out_norm, d, hp.rms_eps, lz.x, s); });
        timed(14 + ph, [&] { launched &= launch_linear(lz, s); });
    }
    if (!launched) {
        set_err("decode: a matrix product was given a fused norm outside its limits");
        return UBD_COMPUTE_FAILED;
    }
    if (!hip_ok(hipGetLastError(), "kernel launch")) return UBD_COMPUTE_FAILED;
    return UBD_OK;
}

// ------------------------------------------------------------------ decode
extern "C" int32_t ubd_decode(ubd_context *ctx, ubd_batch batch) {
    if (!ctx) return UBD_INVALID;
    g_err.clear();
    const double t0 = now_ms();
    if (!hip_ok(hipSetDevice(ctx->model->device), "hipSetDevice")) return UBD_ALLOC_FAILED;
    std::string err;
    const int32_t rc = ctx->planner.decode(batch, ctx, &err);
    if (rc != UBD_OK) {
        if (g_err.empty()) set_err(err);
        if (rc != UBD_NO_KV_SLOT && rc != UBD_INVALID) log_line(2, "decode failed, ret = %d", rc);
        return rc;
    }
    const double dt = now_ms() - t0;
    if (batch.n_tokens > 1) {
        ctx->perf.t_p_eval_ms += dt;
        ctx->perf.n_p_eval += batch.n_tokens;
    } else {
        ctx->perf.t_eval_ms += dt;
        ctx->perf.n_eval += 1;
    }
    ctx->perf.n_decode += 1;
    return UBD_OK;
}

extern "C" int32_t ubd_n_outputs(const ubd_context *ctx) {
    return ctx && ctx->planner.last_ok ? ctx->planner.n_outputs : 0;
}

extern "C" int32_t ubd_synchronize(ubd_context *ctx) {
    if (!ctx) return UBD_INVALID;
    (void)hipSetDevice(ctx->model->device);
    return hip_ok(hipStreamSynchronize(ctx->stream), "synchronize") ? UBD_OK : UBD_COMPUTE_FAILED;
}

namespace {
int32_t resolve_row(const ubd_context *ctx, int32_t i) {
    const Planner &P = ctx->planner;
    if (!P.last_ok || P.n_outputs == 0) return -1;
    if (i < 0) {
        const int32_t r = P.n_outputs + i;
        return r >= 0 && r < P.n_outputs ? r : -1;
    }
    if (i >= (int32_t)P.out_row.size()) return -1;
    return P.out_row[i];
}
}  // namespace

extern "C" float *ubd_get_logits(ubd_context *ctx) {
    if (!ctx || !ctx->planner.last_ok || ctx->planner.n_outputs == 0) return nullptr;
    if (!ctx->logits_host_valid) {
        if (ubd_synchronize(ctx) != UBD_OK) return nullptr;
        const size_t n = (size_t)ctx->planner.n_outputs * ctx->model->hp.n_vocab;
        ctx->logits_host.resize(n);
        if (!hip_ok(hipMemcpy(ctx->logits_host.data(), ctx->logits_dev, n * 4, hipMemcpyDeviceToHost), "logits"))
            return nullptr;
        ctx->logits_host_valid = true;
    }
    return ctx->logits_host.data();
}

extern "C" float *ubd_get_logits_ith(ubd_context *ctx, int32_t i) {
    if (!ctx) return nullptr;
    const int32_t r = resolve_row(ctx, i);
    if (r < 0) return nullptr;
    float *all = ubd_get_logits(ctx);
    return all ? all + (size_t)r * ctx->model->hp.n_vocab : nullptr;
}

extern "C" const float *ubd_get_logits_device(ubd_context *ctx) {
    return ctx && ctx->planner.last_ok && ctx->planner.n_outputs > 0 ? ctx->logits_dev : nullptr;
}

extern "C" ubd_token ubd_sample_greedy(ubd_context *ctx, int32_t i) {
    if (!ctx) return -1;
    const int32_t r = resolve_row(ctx, i);
    if (r < 0) return -1;
    (void)hipSetDevice(ctx->model->device);
    const int V = ctx->model->hp.n_vocab;
    // the kernel writes the pick into pinned host memory: no copy behind it
    launch_argmax(ctx->logits_dev + (size_t)r * V, V, nullptr, 1, V, ctx->argmax_host, ctx->argmax_work, ctx->stream);
    if (!hip_ok(hipStreamSynchronize(ctx->stream), "argmax sync")) return -1;
    return ctx->argmax_host[0];
}

extern "C" int32_t ubd_sample_greedy_all(ubd_context *ctx, ubd_token *out, int32_t cap) {
    if (!ctx || !out) return -1;
    const Planner &P = ctx->planner;
    if (!P.last_ok) return -1;
    if (P.n_outputs > cap) return -1;
    if (P.n_outputs == 0) return 0;
    (void)hipSetDevice(ctx->model->device);
    const int V = ctx->model->hp.n_vocab;
    launch_argmax(ctx->logits_dev, V, nullptr, P.n_outputs, V, ctx->argmax_host, ctx->argmax_work, ctx->stream);
    if (!hip_ok(hipStreamSynchronize(ctx->stream), "argmax sync")) return -1;
    std::memcpy(out, ctx->argmax_host, (size_t)P.n_outputs * 4);
    return P.n_outputs;
}

extern "C" int32_t ubd_greedy_chain(ubd_context *ctx, ubd_token first, ubd_seq_id seq_id, int32_t n_steps,
                                    ubd_token *out) {
    if (!ctx || !out || n_steps < 0) return UBD_INVALID;
    g_err.clear();
    const int V = ctx->model->hp.n_vocab;
    if (first < 0 || first >= V) {
        set_err("ubd_greedy_chain: first token out of range");
        return UBD_INVALID;
    }
    if (!hip_ok(hipSetDevice(ctx->model->device), "hipSetDevice")) return UBD_ALLOC_FAILED;
    int32_t done = 0, rc = UBD_OK;
    while (done < n_steps && rc == UBD_OK) {
        // one block of picks held in pinned memory, then copied out
        const int n = std::min<int32_t>(n_steps - done, UBD_GREEDY_CHAIN_BLOCK);
        int k = 0;
        for (; k < n; ++k) {
            const double t0 = now_ms();
            // steps after the first embed the previous pick, which the argmax
            // kernel leaves in the device token table; 0 stands in for it on
            // the host (a valid id for the batch checks)
            ubd_token tok = done + k == 0 ? first : 0;
            ubd_seq_id sid = seq_id;
            ubd_seq_id *sids = &sid;
            int32_t nsid = 1;
            int8_t lg = 1;
            const ubd_batch b{1, &tok, nullptr, nullptr, &nsid, &sids, &lg};
            ctx->chain_tok = done + k > 0;
            std::string err;
            rc = ctx->planner.decode(b, ctx, &err);
            ctx->chain_tok = false;
            if (rc != UBD_OK) {
                if (g_err.empty()) set_err(err);
                break;
            }
            launch_argmax(ctx->logits_dev, V, nullptr, 1, V, ctx->argmax_host + k, ctx->argmax_work, ctx->stream,
                          ctx->info_dev);
            ctx->perf.t_eval_ms += now_ms() - t0;
            ctx->perf.n_eval += 1;
            ctx->perf.n_decode += 1;
        }
        if (!hip_ok(hipStreamSynchronize(ctx->stream), "greedy chain sync")) return UBD_COMPUTE_FAILED;
        std::memcpy(out + done, ctx->argmax_host, (size_t)k * 4);
        done += k;
    }
    if (rc != UBD_OK && done == 0) return rc;
    return done;
}

// ----------------------------------------------------------------- sampler
struct ubd_sampler {
    ubd_context *ctx = nullptr;
    int device = 0;
    ubd_sampler_params p{};
    std::vector<int32_t> history;
    int32_t *d_hist = nullptr, *d_out = nullptr, *d_ids = nullptr;
    float *d_probs = nullptr;
    int32_t *h_stage = nullptr;     // pinned: history upload, then {token, n}
    int32_t n_last = 0;
};

extern "C" ubd_sampler_params ubd_sampler_default_params(void) {
    ubd_sampler_params p;
    p.top_k = 40;
    p.top_p = 1.f;
    p.min_p = 0.f;
    p.temperature = 1.f;
    p.penalty_last_n = 0;
    p.penalty_repeat = 1.f;
    p.penalty_freq = 0.f;
    p.penalty_present = 0.f;
    return p;
}

extern "C" void ubd_sampler_free(ubd_sampler *s) {
    if (!s) return;
    (void)hipSetDevice(s->device);
    if (s->d_hist) (void)hipFree(s->d_hist);
    if (s->d_out) (void)hipFree(s->d_out);
    if (s->d_ids) (void)hipFree(s->d_ids);
    if (s->d_probs) (void)hipFree(s->d_probs);
    if (s->h_stage) (void)hipHostFree(s->h_stage);
    delete s;
}

extern "C" ubd_sampler *ubd_sampler_init(ubd_context *ctx, ubd_sampler_params p) {
    if (!ctx) {
        set_err("ubd_sampler_init: no context");
        return nullptr;
    }
    if (p.top_k < 1 || p.top_k > SAMPLER_KMAX || !(p.top_p > 0.f && p.top_p <= 1.f) ||
        !(p.min_p >= 0.f && p.min_p < 1.f) || p.penalty_last_n < 0 || p.penalty_last_n > SAMPLER_HMAX ||
        !(p.penalty_repeat > 0.f) || !std::isfinite(p.temperature) || !std::isfinite(p.penalty_freq) ||
        !std::isfinite(p.penalty_present)) {
        set_err("ubd_sampler_init: parameter out of range");
        return nullptr;
    }
    (void)hipSetDevice(ctx->model->device);
    ubd_sampler *s = new ubd_sampler();
    s->ctx = ctx;
    s->device = ctx->model->device;
    s->p = p;
    const bool ok = hip_ok(hipMalloc(&s->d_hist, SAMPLER_HMAX * 4), "sampler alloc") &&
                    hip_ok(hipMalloc(&s->d_out, 2 * 4), "sampler alloc") &&
                    hip_ok(hipMalloc(&s->d_ids, SAMPLER_KMAX * 4), "sampler alloc") &&
                    hip_ok(hipMalloc(&s->d_probs, SAMPLER_KMAX * 4), "sampler alloc") &&
                    hip_ok(hipHostMalloc((void **)&s->h_stage, (SAMPLER_HMAX + 2) * 4, hipHostMallocDefault),
                           "sampler pinned");
    if (!ok) {
        ubd_sampler_free(s);
        return nullptr;
    }
    return s;
}

namespace {
// only the last SAMPLER_HMAX entries are ever read
void remember(ubd_sampler *s, int32_t t) {
    if (s->history.size() >= 16 * SAMPLER_HMAX)
        s->history.erase(s->history.begin(), s->history.end() - SAMPLER_HMAX);
    s->history.push_back(t);
}
}  // namespace

extern "C" void ubd_sampler_accept(ubd_sampler *s, ubd_token t) {
    if (s) remember(s, t);
}

namespace {
ubd_token sampler_run(ubd_sampler *s, const float *logits, int V, float u) {
    ubd_context *ctx = s->ctx;
    (void)hipSetDevice(ctx->model->device);
    const int nh = (int)std::min<size_t>(s->history.size(), (size_t)s->p.penalty_last_n);
    std::copy(s->history.end() - nh, s->history.end(), s->h_stage);
    SamplerArgs a;
    a.logits = logits;
    a.n_vocab = V;
    a.hist = s->d_hist;
    a.n_hist = nh;
    a.top_k = s->p.top_k;
    a.top_p = s->p.top_p;
    a.min_p = s->p.min_p;
    a.temperature = s->p.temperature;
    a.pen_repeat = s->p.penalty_repeat;
    a.pen_freq = s->p.penalty_freq;
    a.pen_present = s->p.penalty_present;
    a.u = u;
    a.out_token = s->d_out;
    a.out_ids = s->d_ids;
    a.out_probs = s->d_probs;
    if ((nh && !hip_ok(hipMemcpyAsync(s->d_hist, s->h_stage, (size_t)nh * 4, hipMemcpyHostToDevice, ctx->stream),
                       "history upload")))
        return -1;
    launch_sampler(a, ctx->stream);
    if (!hip_ok(hipGetLastError(), "sampler") ||
        !hip_ok(hipMemcpyAsync(s->h_stage + SAMPLER_HMAX, s->d_out, 8, hipMemcpyDeviceToHost, ctx->stream), "sample") ||
        !hip_ok(hipStreamSynchronize(ctx->stream), "sample sync"))
        return -1;
    const int32_t tok = s->h_stage[SAMPLER_HMAX];
    s->n_last = s->h_stage[SAMPLER_HMAX + 1];
    remember(s, tok);
    return tok;
}
}  // namespace

extern "C" ubd_token ubd_sampler_sample(ubd_sampler *s, int32_t i, float u) {
    if (!s || !(u >= 0.f && u < 1.f)) return -1;
    const int32_t r = resolve_row(s->ctx, i);
    if (r < 0) return -1;
    const int V = s->ctx->model->hp.n_vocab;
    return sampler_run(s, s->ctx->logits_dev + (size_t)r * V, V, u);
}

extern "C" ubd_token ubd_sampler_sample_logits(ubd_sampler *s, const float *logits, int32_t n_vocab, float u) {
    if (!s || !logits || n_vocab < 1 || !(u >= 0.f && u < 1.f)) return -1;
    return sampler_run(s, logits, n_vocab, u);
}

extern "C" int32_t ubd_sampler_candidates(ubd_sampler *s, ubd_token *ids, float *probs, int32_t cap) {
    if (!s || cap < 0) return -1;
    const int n = std::min(s->n_last, cap);
    if (n > 0 && ((ids && !hip_ok(hipMemcpy(ids, s->d_ids, (size_t)n * 4, hipMemcpyDeviceToHost), "candidates")) ||
                  (probs && !hip_ok(hipMemcpy(probs, s->d_probs, (size_t)n * 4, hipMemcpyDeviceToHost), "candidates"))))
        return -1;
    return s->n_last;
}

// ------------------------------------------------------------------ memory
namespace {
int32_t planner_cells(const Planner &P, int32_t stream, int32_t *pos, uint32_t *seq_words, int32_t cap) {
    if (stream < 0 || (uint32_t)stream >= P.n_stream) return -1;
    const int32_t n = (int32_t)P.n_cells, W = P.cells.n_seq_words();
    if (pos) {
        if (cap < n) return -1;
        std::copy(P.cells.pos_data(stream), P.cells.pos_data(stream) + n, pos);
    }
    if (seq_words) {
        if (cap < n * W) return -1;
        std::copy(P.cells.seq_words(stream), P.cells.seq_words(stream) + (size_t)n * W, seq_words);
    }
    return n;
}
}  // namespace

extern "C" ubd_pos ubd_memory_seq_pos_min(ubd_context *ctx, ubd_seq_id s) {
    return ctx ? ctx->planner.cells.seq_pos_min(s) : -1;
}
extern "C" ubd_pos ubd_memory_seq_pos_max(ubd_context *ctx, ubd_seq_id s) {
    return ctx ? ctx->planner.cells.seq_pos_max(s) : -1;
}
extern "C" bool ubd_memory_seq_rm(ubd_context *ctx, ubd_seq_id s, ubd_pos p0, ubd_pos p1) {
    if (!ctx) return false;
    (void)hipSetDevice(ctx->model->device);
    return ctx->planner.seq_rm(s, p0, p1, ctx);
}

extern "C" bool ubd_memory_seq_cp(ubd_context *ctx, ubd_seq_id src, ubd_seq_id dst, ubd_pos p0, ubd_pos p1) {
    if (!ctx) return false;
    (void)hipSetDevice(ctx->model->device);
    return ctx->planner.seq_cp(src, dst, p0, p1, ctx);
}

extern "C" bool ubd_memory_seq_keep(ubd_context *ctx, ubd_seq_id s) {
    if (!ctx) return false;
    (void)hipSetDevice(ctx->model->device);
    return ctx->planner.seq_keep(s, ctx);
}

extern "C" int32_t ubd_memory_defrag(ubd_context *ctx) {
    if (!ctx) return UBD_INVALID;
    (void)hipSetDevice(ctx->model->device);
    return ctx->planner.defrag(ctx);
}

extern "C" int32_t ubd_memory_cells(ubd_context *ctx, int32_t stream, int32_t *pos, uint32_t *seq_words,
                                    int32_t cap) {
    if (!ctx) return -1;
    return planner_cells(ctx->planner, stream, pos, seq_words, cap);
}

extern "C" int32_t ubd_get_kv_cells(ubd_context *ctx, int32_t *cells_out, int32_t cap) {
    if (!ctx || !ctx->planner.last_ok) return -1;
    const auto &c = ctx->planner.cell_of;
    if ((int32_t)c.size() > cap || !cells_out) return -1;
    std::copy(c.begin(), c.end(), cells_out);
    return (int32_t)c.size();
}

extern "C" int32_t ubd_kv_fill(ubd_context *ctx, ubd_seq_id s, int32_t n_pos, const void *const *k_layers,
                               const void *const *v_layers, ubd_type src_type, int32_t on_device) {
    if (!ctx || !k_layers || !v_layers || n_pos <= 0) return UBD_INVALID;
    if (s < 0 || (uint32_t)s >= ctx->planner.n_seq_max) return UBD_INVALID;
    if (src_type != UBD_TYPE_F16 && src_type != UBD_TYPE_F32) return UBD_INVALID;
    (void)hipSetDevice(ctx->model->device);
    const ubd_hparams &hp = ctx->model->hp;
    const int hd = ctx->model->head_dim, Hk = hp.n_head_kv;
    const int st = ctx->planner.cells.stream_of(s);
    std::vector<int32_t> cells;
    if (ctx->planner.cells.seq_pos_max(s) >= 0) return UBD_INVALID;
    if (!ctx->planner.cells.fill_sequence(s, n_pos, &cells)) return UBD_NO_KV_SLOT;
    const size_t rows_bytes = (size_t)n_pos * Hk * hd * (src_type == UBD_TYPE_F32 ? 4 : 2);
    int32_t *dcells = nullptr;
    void *stage = nullptr;
    bool ok = hip_ok(hipMalloc(&dcells, cells.size() * 4), "kv_fill alloc") &&
              hip_ok(hipMemcpy(dcells, cells.data(), cells.size() * 4, hipMemcpyHostToDevice), "kv_fill cells");
    if (ok && !on_device) ok = hip_ok(hipMalloc(&stage, rows_bytes), "kv_fill staging");
    const int srct = src_type == UBD_TYPE_F32 ? KV_F32 : KV_F16;
    for (int il = 0; ok && il < hp.n_layer; ++il) {
        for (int which = 0; ok && which < 2; ++which) {
            const void *src = which == 0 ? k_layers[il] : v_layers[il];
            if (!src) {
                ok = false;
                set_err("kv_fill: missing layer array");
                break;
            }
            if (!on_device) {
                ok = hip_ok(hipMemcpyAsync(stage, src, rows_bytes, hipMemcpyHostToDevice, ctx->stream), "kv upload");
                src = stage;
            }
            void *cache = which == 0 ? (char *)ctx->k_cache + ctx->k_layer_bytes * il
                                     : (char *)ctx->v_cache + ctx->v_layer_bytes * il;
            const int ct = which == 0 ? ctx->type_k : ctx->type_v;
            if (ct == KV_Q8)
                launch_kv_quant(src, srct, Hk * hd, n_pos, dcells, nullptr, st, cache, which == 1, Hk, hd,
                                (int)ctx->cell_stride, ctx->kv_layer_elems, ctx->stream);
            else
                launch_kv_store(src, srct, n_pos, dcells, cache, ct, which == 1, st, Hk, hd, (int)ctx->cell_stride,
                                ctx->stream);
            ok = ok && hip_ok(hipGetLastError(), "kv_store");
            if (!on_device) ok = ok && hip_ok(hipStreamSynchronize(ctx->stream), "kv sync");
        }
    }
    ok = ok && hip_ok(hipStreamSynchronize(ctx->stream), "kv sync") && ctx->sync_cell_tables(st);
    if (dcells) (void)hipFree(dcells);
    if (stage) (void)hipFree(stage);
    if (!ok) {
        ctx->planner.seq_rm(s, -1, -1, ctx);
        return UBD_INVALID;
    }
    return UBD_OK;
}

extern "C" int32_t ubd_kv_read(ubd_context *ctx, int32_t layer, int32_t stream, int32_t which, int32_t cell0,
                               int32_t n, float *out) {
    if (!ctx || !out || n <= 0) return UBD_INVALID;
    const ubd_hparams &hp = ctx->model->hp;
    const Planner &P = ctx->planner;
    if (layer < 0 || layer >= hp.n_layer || stream < 0 || (uint32_t)stream >= P.n_stream || cell0 < 0 ||
        (uint32_t)(cell0 + n) > P.n_cells || (which != 0 && which != 1))
        return UBD_INVALID;
    (void)hipSetDevice(ctx->model->device);
    const int hd = ctx->model->head_dim, Hk = hp.n_head_kv;
    const size_t bytes = (size_t)n * Hk * hd * 4;
    float *tmp = nullptr;
    if (!hip_ok(hipMalloc(&tmp, bytes), "kv_read alloc")) return UBD_ALLOC_FAILED;
    const void *cache = which == 0 ? (const char *)ctx->k_cache + ctx->k_layer_bytes * layer
                                   : (const char *)ctx->v_cache + ctx->v_layer_bytes * layer;
    launch_kv_load(cache, which == 0 ? ctx->type_k : ctx->type_v, which == 1, stream, cell0, n, Hk, hd,
                   (int)ctx->cell_stride, ctx->kv_layer_elems, tmp, ctx->stream);
    bool ok = hip_ok(hipGetLastError(), "kv_load") && hip_ok(hipStreamSynchronize(ctx->stream), "kv_read sync") &&
              hip_ok(hipMemcpy(out, tmp, bytes, hipMemcpyDeviceToHost), "kv_read copy");
    (void)hipFree(tmp);
    return ok ? UBD_OK : UBD_COMPUTE_FAILED;
}

// ------------------------------------------------------------- diagnostics
extern "C" int32_t ubd_debug_keep_residuals(ubd_context *ctx, int32_t enable) {
    if (!ctx) return UBD_INVALID;
    if (!enable) {
        ctx->dump = nullptr;   // the block stays with the context's allocations
        return UBD_OK;
    }
    if (ctx->dump) return UBD_OK;
    const ubd_hparams &hp = ctx->model->hp;
    (void)hipSetDevice(ctx->model->device);
    ctx->dump = (float *)ctx->mem.get((size_t)(hp.n_layer + 1) * ctx->cap * hp.n_embd * 4);
    return ctx->dump ? UBD_OK : UBD_ALLOC_FAILED;
}

extern "C" int32_t ubd_debug_get_residual(ubd_context *ctx, int32_t layer, float *out, int32_t cap_tokens) {
    if (!ctx || !ctx->dump || !out) return -1;
    const ubd_hparams &hp = ctx->model->hp;
    if (layer < 0 || layer > hp.n_layer) return -1;
    const int32_t T = (int32_t)ctx->last_ub_idx.size();
    if (T > cap_tokens) return -1;
    if (ubd_synchronize(ctx) != UBD_OK) return -1;
    if (!hip_ok(hipMemcpy(out, ctx->dump + (size_t)layer * ctx->cap * hp.n_embd, (size_t)T * hp.n_embd * 4,
                          hipMemcpyDeviceToHost), "residual copy"))
        return -1;
    return T;
}

extern "C" int32_t ubd_debug_last_ubatch(ubd_context *ctx, int32_t *batch_idx, int32_t cap) {
    if (!ctx || !batch_idx) return -1;
    const int32_t T = (int32_t)ctx->last_ub_idx.size();
    if (T > cap) return -1;
    std::copy(ctx->last_ub_idx.begin(), ctx->last_ub_idx.end(), batch_idx);
    return T;
}

static const char *kClassNames[UBD_KERNEL_CLASSES] = {
    "decode.embed",       "prefill.embed",       "decode.rmsnorm",     "prefill.rmsnorm",
    "decode.qkv",         "prefill.qkv",         "decode.attention",   "prefill.attention",
    "decode.attn_output", "prefill.attn_output", "decode.ffn_gate_up", "prefill.ffn_gate_up",
    "decode.ffn_down",    "prefill.ffn_down",    "decode.logits",      "prefill.logits"};

extern "C" int32_t ubd_debug_kernel_timing(ubd_context *ctx, uint32_t mask) {
    if (!ctx) return UBD_INVALID;
    ctx->collect_timing();
    ctx->time_mask = mask;
    return UBD_OK;
}

extern "C" const char *ubd_debug_kernel_class_name(int32_t cls) {
    return cls >= 0 && cls < UBD_KERNEL_CLASSES ? kClassNames[cls] : "";
}

extern "C" int32_t ubd_debug_kernel_stats(ubd_context *ctx, int32_t *launches, double *total_ms, int32_t n) {
    if (!ctx || n < 0 || n > UBD_KERNEL_CLASSES) return UBD_INVALID;
    (void)hipSetDevice(ctx->model->device);
    ctx->collect_timing();
    for (int32_t i = 0; i < n; ++i) {
        if (launches) launches[i] = ctx->t_launches[i];
        if (total_ms) total_ms[i] = ctx->t_ms[i];
        ctx->t_launches[i] = 0;
        ctx->t_ms[i] = 0;
    }
    return n;
}

extern "C" void ubd_perf_get(const ubd_context *ctx, ubd_perf *out) {
    if (!ctx || !out) return;
    *out = ctx->perf;
    out->t_load_ms = ctx->model->t_load_ms;
}

extern "C" void ubd_perf_reset(ubd_context *ctx) {
    if (ctx) ctx->perf = ubd_perf{};
}

extern "C" int32_t ubd_debug_set_tuning(const char *key, int32_t value) {
    if (!key) return UBD_INVALID;
    const std::string k(key);
    if (k == "skinny_nw") {
        g_tuning.skinny_nw = value;
    } else if (k == "fuse_norm") {
        g_tuning.fuse_norm = value;
    } else if (k == "post_norm") {
        g_tuning.post_norm = value;
    } else if (k == "attn_chunk_min") {
        g_tuning.attn_chunk_min = value;
    } else if (k == "attn_pair") {
        g_tuning.attn_pair = value;
    } else if (k == "attn_nt_mb") {
        g_tuning.attn_nt_mb = value;
    } else if (k == "gemm_wpd") {
        g_tuning.gemm_wpd = value;
    } else if (k == "gemm_deep") {
        g_tuning.gemm_deep = value;
    } else if (k == "act_tiled") {
        g_tuning.act_tiled = value;
    } else if (k == "prefill_lo") {
        g_tuning.prefill_lo = value;
    } else if (k == "ldsx") {
        g_tuning.ldsx = value;
    } else if (k == "ldsx_early") {
        g_tuning.ldsx_early = value;
    } else if (k == "gemm") {
        g_tuning.gemm = value;
    } else if (k == "gemm_split") {
        g_tuning.gemm_split = value;
    } else if (k == "gemm_shape") {
        g_tuning.gemm_shape = value;
    } else if (k == "small_rb") {
        g_tuning.small_rb = value;
    } else {
        return UBD_INVALID;
    }
    ++g_tuning_gen;
    return UBD_OK;
}

extern "C" void ubd_log_set(ubd_log_fn fn, void *user_data) {
    g_log = fn;
    g_log_ud = user_data;
}

extern "C" const char *ubd_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------------- batch
extern "C" ubd_batch ubd_batch_init(int32_t n_tokens_alloc, int32_t embd, int32_t n_seq_max) {
    ubd_batch b{};
    if (n_tokens_alloc <= 0 || embd != 0 || n_seq_max <= 0) return b;
    const size_t n = (size_t)n_tokens_alloc;
    b.token = (ubd_token *)calloc(n, sizeof(ubd_token));
    b.pos = (ubd_pos *)calloc(n, sizeof(ubd_pos));
    b.n_seq_id = (int32_t *)calloc(n, sizeof(int32_t));
    b.seq_id = (ubd_seq_id **)calloc(n + 1, sizeof(ubd_seq_id *));
    b.logits = (int8_t *)calloc(n, 1);
    for (size_t i = 0; i < n; ++i) b.seq_id[i] = (ubd_seq_id *)calloc((size_t)n_seq_max, sizeof(ubd_seq_id));
    return b;
}

extern "C" void ubd_batch_free(ubd_batch b) {
    if (b.seq_id) {
        for (size_t i = 0; b.seq_id[i]; ++i) free(b.seq_id[i]);
        free(b.seq_id);
    }
    free(b.token);
    free(b.pos);
    free(b.n_seq_id);
    free(b.logits);
}

extern "C" ubd_batch ubd_batch_get_one(ubd_token *tokens, int32_t n_tokens) {
    ubd_batch b{};
    b.n_tokens = n_tokens;
    b.token = tokens;
    return b;
}

// ------------------------------------------------------- host-only planner
struct ubd_planner {
    Planner p;
};

namespace {
struct StubExecutor : Executor {
    int32_t fail_at = -1, fail_code = UBD_OK;
    int32_t run_ubatch(const UBatch &, int32_t k) override { return k == fail_at ? fail_code : UBD_OK; }
};
}  // namespace

extern "C" ubd_planner *ubd_planner_new(uint32_t n_ctx, uint32_t n_batch, uint32_t n_ubatch, uint32_t n_seq_max,
                                        bool kv_unified, int32_t n_vocab) {
    ubd_planner *pl = new ubd_planner();
    std::string err;
    if (pl->p.init(n_ctx, n_batch, n_ubatch, n_seq_max, kv_unified, n_vocab, &err) != UBD_OK) {
        set_err(err);
        delete pl;
        return nullptr;
    }
    return pl;
}

extern "C" void ubd_planner_free(ubd_planner *p) { delete p; }

extern "C" int32_t ubd_planner_decode(ubd_planner *p, ubd_batch batch, int32_t fail_at, int32_t fail_code) {
    if (!p) return UBD_INVALID;
    StubExecutor ex;
    ex.fail_at = fail_at;
    ex.fail_code = fail_code;
    std::string err;
    return p->p.decode(batch, &ex, &err);
}

extern "C" int32_t ubd_planner_n_ubatches(const ubd_planner *p) { return p ? (int32_t)p->p.ubatches.size() : -1; }

extern "C" int32_t ubd_planner_ubatch(const ubd_planner *p, int32_t k, int32_t *batch_idx, int32_t *cells,
                                      int32_t *streams, int32_t cap) {
    if (!p || k < 0 || k >= (int32_t)p->p.ubatches.size()) return -1;
    const UBatch &ub = p->p.ubatches[k];
    if (ub.size() > cap) return -1;
    for (int32_t t = 0; t < ub.size(); ++t) {
        if (batch_idx) batch_idx[t] = ub.idx[t];
        if (cells) cells[t] = ub.cell[t];
        if (streams) streams[t] = ub.stream[t];
    }
    return ub.size();
}

extern "C" int32_t ubd_planner_output_row(const ubd_planner *p, int32_t i) {
    if (!p || i < 0 || i >= (int32_t)p->p.out_row.size()) return -1;
    return p->p.out_row[i];
}

extern "C" int32_t ubd_planner_n_outputs(const ubd_planner *p) { return p && p->p.last_ok ? p->p.n_outputs : 0; }

extern "C" ubd_pos ubd_planner_seq_pos_min(const ubd_planner *p, ubd_seq_id s) {
    return p ? p->p.cells.seq_pos_min(s) : -1;
}
extern "C" ubd_pos ubd_planner_seq_pos_max(const ubd_planner *p, ubd_seq_id s) {
    return p ? p->p.cells.seq_pos_max(s) : -1;
}
extern "C" bool ubd_planner_seq_rm(ubd_planner *p, ubd_seq_id s, ubd_pos p0, ubd_pos p1) {
    return p ? p->p.seq_rm(s, p0, p1, nullptr) : false;
}
extern "C" bool ubd_planner_seq_cp(ubd_planner *p, ubd_seq_id src, ubd_seq_id dst, ubd_pos p0, ubd_pos p1) {
    return p ? p->p.seq_cp(src, dst, p0, p1, nullptr) : false;
}
extern "C" bool ubd_planner_seq_keep(ubd_planner *p, ubd_seq_id s) { return p ? p->p.seq_keep(s, nullptr) : false; }
extern "C" int32_t ubd_planner_defrag(ubd_planner *p) {
    return p ? p->p.defrag(nullptr) : UBD_INVALID;
}
extern "C" int32_t ubd_planner_cells(const ubd_planner *p, int32_t stream, int32_t *pos, uint32_t *seq_words,
                                     int32_t cap) {
    return p ? planner_cells(p->p, stream, pos, seq_words, cap) : -1;
}
extern "C" int32_t ubd_planner_n_kv(const ubd_planner *p, int32_t stream) {
    if (!p || stream < 0 || (uint32_t)stream >= p->p.n_stream) return -1;
    return p->p.cells.n_kv(stream);
}
