// GGUF reader and the model load from GGUF files; see gguf.h for the
// pages it follows.
#include "gguf.h"

#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <memory>

#include "common.h"
#include "ubd.h"

namespace ubd {

bool gguf_type_size(int32_t type, uint64_t *block_bytes, uint64_t *block_values) {
    switch (type) {
    case GT_F32: *block_bytes = 4; *block_values = 1; return true;
    case GT_F16: *block_bytes = 2; *block_values = 1; return true;
    case GT_BF16: *block_bytes = 2; *block_values = 1; return true;
    case GT_Q8_0: *block_bytes = 34; *block_values = 32; return true;
    default: return false;
    }
}

const char *gguf_type_name(int32_t type) {
    switch (type) {
    case GT_F32: return "F32";
    case GT_F16: return "F16";
    case GT_BF16: return "BF16";
    case GT_Q8_0: return "Q8_0";
    default: return "?";
    }
}

namespace {

// Sequential reads from a file through a buffer; every read is checked
// against the file size.
class Reader {
public:
    Reader(int fd, uint64_t size) : fd_(fd), size_(size) {}
    uint64_t at() const { return pos_; }
    uint64_t left() const { return size_ - pos_; }
    bool take(void *dst, uint64_t n) {
        if (n > left()) return false;
        uint8_t *d = (uint8_t *)dst;
        while (n > 0) {
            if (pos_ < buf_at_ || pos_ >= buf_at_ + buf_.size()) {
                buf_.resize((size_t)std::min<uint64_t>(1 << 20, size_ - pos_));
                buf_at_ = pos_;
                size_t got = 0;
                while (got < buf_.size()) {
                    const ssize_t r = pread(fd_, buf_.data() + got, buf_.size() - got, (off_t)(pos_ + got));
                    if (r <= 0) return false;
                    got += (size_t)r;
                }
            }
            const uint64_t off = pos_ - buf_at_;
            const uint64_t k = std::min<uint64_t>(n, buf_.size() - off);
            if (d) std::memcpy(d, buf_.data() + off, (size_t)k);
            if (d) d += k;
            pos_ += k;
            n -= k;
        }
        return true;
    }
    template <typename T> bool get(T *v) { return take(v, sizeof(T)); }
    bool str(std::string *s) {
        uint64_t n = 0;
        if (!get(&n) || n > left()) return false;
        s->resize((size_t)n);
        return take(&(*s)[0], n);
    }

private:
    int fd_;
    uint64_t size_, pos_ = 0, buf_at_ = 0;
    std::vector<uint8_t> buf_;
};

int scalar_bytes(int32_t t) {
    switch (t) {
    case GV_U8: case GV_I8: case GV_BOOL: return 1;
    case GV_U16: case GV_I16: return 2;
    case GV_U32: case GV_I32: case GV_F32: return 4;
    case GV_U64: case GV_I64: case GV_F64: return 8;
    default: return 0;
    }
}

// One scalar into v (appended to the vector of its kind).
bool read_scalar(Reader &r, int32_t t, GgufValue *v) {
    uint8_t b[8] = {0};
    const int n = scalar_bytes(t);
    if (!n || !r.take(b, (uint64_t)n)) return false;
    int64_t i = 0;
    double f = 0;
    switch (t) {
    case GV_U8: i = b[0]; break;
    case GV_I8: i = (int8_t)b[0]; break;
    case GV_BOOL: i = b[0] != 0; break;
    case GV_U16: { uint16_t x; std::memcpy(&x, b, 2); i = x; break; }
    case GV_I16: { int16_t x; std::memcpy(&x, b, 2); i = x; break; }
    case GV_U32: { uint32_t x; std::memcpy(&x, b, 4); i = x; break; }
    case GV_I32: { int32_t x; std::memcpy(&x, b, 4); i = x; break; }
    case GV_U64: { uint64_t x; std::memcpy(&x, b, 8); i = (int64_t)x; break; }
    case GV_I64: { int64_t x; std::memcpy(&x, b, 8); i = x; break; }
    case GV_F32: { float x; std::memcpy(&x, b, 4); f = x; break; }
    case GV_F64: { double x; std::memcpy(&x, b, 8); f = x; break; }
    default: return false;
    }
    if (t == GV_F32 || t == GV_F64)
        v->f.push_back(f);
    else
        v->i.push_back(i);
    return true;
}

bool read_value(Reader &r, int32_t t, GgufValue *v, int depth) {
    if (t == GV_STR) {
        std::string s;
        if (!r.str(&s)) return false;
        v->s.push_back(std::move(s));
        return true;
    }
    if (t != GV_ARR) return read_scalar(r, t, v);
    if (depth > 4) return false;
    uint32_t et = 0;
    uint64_t n = 0;
    if (!r.get(&et) || !r.get(&n)) return false;
    const int32_t e = (int32_t)et;
    // every element takes at least this many bytes: bound n by the file
    const uint64_t least = e == GV_STR ? 8 : e == GV_ARR ? 12 : (uint64_t)scalar_bytes(e);
    if (least == 0 || n > r.left() / least) return false;
    if (depth == 0) {
        v->etype = e;
        v->n = n;
        for (uint64_t k = 0; k < n; ++k)
            if (!read_value(r, e, v, depth + 1)) return false;
        return true;
    }
    GgufValue skip;      // nested arrays: parsed for validity, kept as counts only
    for (uint64_t k = 0; k < n; ++k)
        if (!read_value(r, e, &skip, depth + 1)) return false;
    return true;
}

}  // namespace

GgufFile::~GgufFile() {
    if (map_) munmap(map_, (size_t)file_size);
    if (fd_ >= 0) close(fd_);
}

bool GgufFile::open(const std::string &p, std::string *err) {
    auto bad = [&](const std::string &m) {
        if (err) *err = p + ": " + m;
        return false;
    };
    path = p;
    fd_ = ::open(p.c_str(), O_RDONLY | O_CLOEXEC);
    if (fd_ < 0) return bad("cannot open");
    struct stat st {};
    if (fstat(fd_, &st) != 0) return bad("cannot stat");
    file_size = (uint64_t)st.st_size;
    Reader r(fd_, file_size);
    char magic[4];
    if (!r.take(magic, 4) || std::memcmp(magic, "GGUF", 4) != 0) return bad("not a GGUF file");
    uint64_t n_tensors = 0, n_kv = 0;
    if (!r.get(&version)) return bad("truncated file");
    if (version != 3) return bad("unsupported GGUF version " + std::to_string(version));
    if (!r.get(&n_tensors) || !r.get(&n_kv)) return bad("truncated file");
    // a key takes at least 12 bytes, a tensor record at least 32
    if (n_kv > r.left() / 12 || n_tensors > r.left() / 32) return bad("truncated file");
    for (uint64_t k = 0; k < n_kv; ++k) {
        std::string key;
        uint32_t t = 0;
        if (!r.str(&key) || !r.get(&t)) return bad("truncated file");
        GgufValue v;
        v.type = (int32_t)t;
        if (v.type < 0 || v.type > GV_F64) return bad("unknown value type for key " + key);
        if (!read_value(r, v.type, &v, 0)) return bad("bad or truncated value for key " + key);
        if (key_index.count(key)) return bad("duplicate key " + key);
        key_index[key] = (int64_t)keys.size();
        keys.push_back(key);
        values.push_back(std::move(v));
    }
    int64_t al = 32;
    if (find("general.alignment") && !get_int("general.alignment", &al)) return bad("bad general.alignment");
    if (al <= 0 || (al & (al - 1))) return bad("alignment must be a power of two");
    alignment = (uint64_t)al;
    for (uint64_t k = 0; k < n_tensors; ++k) {
        GgufTensor t;
        uint32_t nd = 0, ty = 0;
        if (!r.str(&t.name) || !r.get(&nd)) return bad("truncated file");
        if (nd < 1 || nd > 4) return bad("tensor " + t.name + ": " + std::to_string(nd) + " dimensions");
        t.n_dims = (int32_t)nd;
        uint64_t n = 1;
        for (uint32_t d = 0; d < nd; ++d) {
            uint64_t x = 0;
            if (!r.get(&x)) return bad("truncated file");
            if (x == 0 || x > (uint64_t)INT64_MAX || n > (uint64_t)INT64_MAX / x)
                return bad("tensor " + t.name + ": bad dimensions");
            t.ne[d] = (int64_t)x;
            n *= x;
        }
        if (!r.get(&ty) || !r.get(&t.offset)) return bad("truncated file");
        t.type = (int32_t)ty;
        uint64_t bb = 0, bv = 0;
        if (!gguf_type_size(t.type, &bb, &bv)) return bad("tensor " + t.name + ": unknown type " + std::to_string(ty));
        if ((uint64_t)t.ne[0] % bv) return bad("tensor " + t.name + ": rows not a whole number of blocks");
        t.nbytes = n / bv * bb;
        if (t.offset % alignment) return bad("tensor " + t.name + ": misaligned offset");
        if (tensor_index.count(t.name)) return bad("tensor " + t.name + " is duplicated");
        tensor_index[t.name] = (int64_t)tensors.size();
        tensors.push_back(std::move(t));
    }
    data_start = (r.at() + alignment - 1) / alignment * alignment;
    for (const GgufTensor &t : tensors)
        if (t.offset > file_size || t.nbytes > file_size - t.offset || data_start > file_size - t.offset - t.nbytes)
            return bad("tensor " + t.name + ": data past the end of the file");
    return true;
}

const uint8_t *GgufFile::map(std::string *err) {
    if (map_) return map_;
    void *p = mmap(nullptr, (size_t)file_size, PROT_READ, MAP_PRIVATE, fd_, 0);
    if (p == MAP_FAILED) {
        if (err) *err = path + ": mmap failed";
        return nullptr;
    }
    map_ = (uint8_t *)p;
    return map_;
}

bool GgufFile::read(const GgufTensor &t, void *dst, std::string *err) const {
    uint8_t *d = (uint8_t *)dst;
    uint64_t done = 0;
    while (done < t.nbytes) {
        const ssize_t r = pread(fd_, d + done, (size_t)std::min<uint64_t>(t.nbytes - done, 1u << 30),
                                (off_t)(data_start + t.offset + done));
        if (r <= 0) {
            if (err) *err = path + ": read failed for " + t.name;
            return false;
        }
        done += (uint64_t)r;
    }
    return true;
}

const GgufValue *GgufFile::find(const std::string &key) const {
    auto it = key_index.find(key);
    return it == key_index.end() ? nullptr : &values[(size_t)it->second];
}

bool GgufFile::get_int(const std::string &key, int64_t *out) const {
    const GgufValue *v = find(key);
    if (!v || v->type == GV_ARR || v->i.empty()) return false;
    *out = v->i[0];
    return true;
}

bool GgufFile::get_float(const std::string &key, double *out) const {
    const GgufValue *v = find(key);
    if (!v || v->type == GV_ARR) return false;
    if (!v->f.empty()) {
        *out = v->f[0];
        return true;
    }
    if (!v->i.empty()) {
        *out = (double)v->i[0];
        return true;
    }
    return false;
}

bool GgufFile::get_str(const std::string &key, std::string *out) const {
    const GgufValue *v = find(key);
    if (!v || v->type != GV_STR) return false;
    *out = v->s[0];
    return true;
}

namespace {

// Paths of all parts of a split model from the first part's path
// ("<prefix>-00001-of-0000N.gguf", the loading page's naming).
bool split_paths(const GgufFile &first, std::vector<std::string> *out, std::string *err) {
    out->assign(1, first.path);
    int64_t count = 1;
    if (!first.find("split.count")) return true;
    if (!first.get_int("split.count", &count) || count < 1 || count > 99999) {
        *err = first.path + ": bad split.count";
        return false;
    }
    if (count == 1) return true;
    char tail[32];
    std::snprintf(tail, sizeof tail, "-%05d-of-%05d.gguf", 1, (int)count);
    const std::string &p = first.path;
    if (p.size() < std::strlen(tail) || p.compare(p.size() - std::strlen(tail), std::string::npos, tail) != 0) {
        *err = p + ": a split model's first part must be named <prefix>" + tail;
        return false;
    }
    const std::string prefix = p.substr(0, p.size() - std::strlen(tail));
    for (int64_t k = 2; k <= count; ++k) {
        std::snprintf(tail, sizeof tail, "-%05d-of-%05d.gguf", (int)k, (int)count);
        out->push_back(prefix + tail);
    }
    return true;
}

struct GgufModel {
    std::vector<std::unique_ptr<GgufFile>> files;
    std::map<std::string, std::pair<const GgufFile *, const GgufTensor *>> where;
    ubd_hparams hp{};
};

bool open_model(const char *path, GgufModel *m, std::string *err) {
    auto first = std::make_unique<GgufFile>();
    if (!first->open(path, err)) return false;
    std::vector<std::string> paths;
    if (!split_paths(*first, &paths, err)) return false;
    m->files.push_back(std::move(first));
    for (size_t k = 1; k < paths.size(); ++k) {
        auto f = std::make_unique<GgufFile>();
        if (!f->open(paths[k], err)) return false;
        int64_t no = -1;
        if (!f->get_int("split.no", &no) || no != (int64_t)k) {
            *err = paths[k] + ": split.no does not match its place";
            return false;
        }
        m->files.push_back(std::move(f));
    }
    for (const auto &f : m->files)
        for (const GgufTensor &t : f->tensors) {
            if (m->where.count(t.name)) {
                *err = "invalid model: tensor " + t.name + " is duplicated";
                return false;
            }
            m->where[t.name] = {f.get(), &t};
        }
    int64_t total = 0;
    if (m->files[0]->get_int("split.tensors.count", &total) && total != (int64_t)m->where.size()) {
        *err = "split.tensors.count does not match the tensors found";
        return false;
    }
    // hyperparameters from the architecture-prefixed keys ([ENG] Step 4)
    const GgufFile &g = *m->files[0];
    std::string arch;
    if (!g.get_str("general.architecture", &arch) || arch != "llama") {
        *err = "unsupported architecture '" + arch + "' (only llama)";
        return false;
    }
    auto need = [&](const char *k, int64_t *v) {
        if (g.get_int(std::string("llama.") + k, v)) return true;
        *err = std::string("missing or non-integer key llama.") + k;
        return false;
    };
    int64_t n_layer, n_embd, n_head, n_ff, n_ctx, n_head_kv;
    double eps = 0, base = 10000.0;
    if (!need("block_count", &n_layer) || !need("embedding_length", &n_embd) ||
        !need("attention.head_count", &n_head) || !need("feed_forward_length", &n_ff) ||
        !need("context_length", &n_ctx))
        return false;
    if (!g.get_int("llama.attention.head_count_kv", &n_head_kv)) n_head_kv = n_head;
    if (!g.get_float("llama.attention.layer_norm_rms_epsilon", &eps)) {
        *err = "missing key llama.attention.layer_norm_rms_epsilon";
        return false;
    }
    if (g.find("llama.rope.freq_base") && !g.get_float("llama.rope.freq_base", &base)) {
        *err = "bad key llama.rope.freq_base";
        return false;
    }
    auto emb = m->where.find("token_embd.weight");
    if (emb == m->where.end() || emb->second.second->n_dims != 2) {
        *err = "missing or malformed token_embd.weight";
        return false;
    }
    const int64_t lim = 1 << 30;
    for (int64_t v : {n_layer, n_embd, n_head, n_ff, n_ctx, n_head_kv, emb->second.second->ne[1]})
        if (v <= 0 || v > lim) {
            *err = "hyperparameter out of range";
            return false;
        }
    ubd_hparams &hp = m->hp;
    hp.n_layer = (int32_t)n_layer;
    hp.n_embd = (int32_t)n_embd;
    hp.n_head = (int32_t)n_head;
    hp.n_head_kv = (int32_t)n_head_kv;
    hp.n_ff = (int32_t)n_ff;
    hp.n_vocab = (int32_t)emb->second.second->ne[1];
    hp.n_ctx_train = (int32_t)n_ctx;
    hp.rms_eps = (float)eps;
    hp.rope_freq_base = (float)base;
    hp.rope_type = 0;
    return true;
}

void info_of(const GgufModel &m, ubd_gguf_info *info) {
    std::map<int32_t, int64_t> counts;
    double params = 0, bytes = 0;
    int64_t n = 0;
    for (const auto &f : m.files) {
        bytes += (double)f->file_size;
        for (const GgufTensor &t : f->tensors) {
            double e = 1;
            for (int d = 0; d < t.n_dims; ++d) e *= (double)t.ne[d];
            params += e;
            counts[t.type] += 1;
            ++n;
        }
    }
    int32_t top = -1;
    int64_t best = -1;
    for (auto &kv : counts)
        if (kv.second > best) {
            best = kv.second;
            top = kv.first;
        }
    info->version = m.files[0]->version;
    info->n_files = (int32_t)m.files.size();
    info->n_tensors = n;
    info->n_params = params;
    info->file_bytes = bytes;
    info->bpw = params > 0 ? bytes * 8.0 / params : 0.0;
    info->file_type = top;
    info->all_same = counts.size() == 1 ? 1 : 0;
    info->hparams = m.hp;
}

}  // namespace
}  // namespace ubd

using namespace ubd;

// ------------------------------------------------------------------ C ABI
struct ubd_gguf {
    GgufFile f;
};

extern "C" ubd_gguf *ubd_gguf_open(const char *path, int32_t *status) {
    if (!path) {
        if (status) *status = UBD_INVALID;
        return nullptr;
    }
    auto *g = new ubd_gguf();
    std::string err;
    if (!g->f.open(path, &err)) {
        set_error(err);
        delete g;
        if (status) *status = UBD_INVALID;
        return nullptr;
    }
    if (status) *status = UBD_OK;
    return g;
}

extern "C" void ubd_gguf_close(ubd_gguf *g) { delete g; }
extern "C" uint32_t ubd_gguf_version(const ubd_gguf *g) { return g ? g->f.version : 0; }
extern "C" int64_t ubd_gguf_n_kv(const ubd_gguf *g) { return g ? (int64_t)g->f.keys.size() : -1; }
extern "C" int64_t ubd_gguf_data_offset(const ubd_gguf *g) { return g ? (int64_t)g->f.data_start : -1; }

namespace {
const GgufValue *value_at(const ubd_gguf *g, int64_t i) {
    return g && i >= 0 && i < (int64_t)g->f.values.size() ? &g->f.values[(size_t)i] : nullptr;
}
const GgufTensor *tensor_at(const ubd_gguf *g, int64_t i) {
    return g && i >= 0 && i < (int64_t)g->f.tensors.size() ? &g->f.tensors[(size_t)i] : nullptr;
}
// element j of a value: j < 0 = the scalar itself
bool elem_ok(const GgufValue *v, int64_t j) {
    if (!v) return false;
    if (v->type == GV_ARR) return j >= 0 && (uint64_t)j < v->n && v->etype != GV_ARR;
    return j < 0;
}
}  // namespace

extern "C" int64_t ubd_gguf_find_key(const ubd_gguf *g, const char *key) {
    if (!g || !key) return -1;
    auto it = g->f.key_index.find(key);
    return it == g->f.key_index.end() ? -1 : it->second;
}
extern "C" const char *ubd_gguf_key(const ubd_gguf *g, int64_t i) {
    return value_at(g, i) ? g->f.keys[(size_t)i].c_str() : nullptr;
}
extern "C" int32_t ubd_gguf_kv_type(const ubd_gguf *g, int64_t i) {
    const GgufValue *v = value_at(g, i);
    return v ? v->type : -1;
}
extern "C" int32_t ubd_gguf_arr_type(const ubd_gguf *g, int64_t i) {
    const GgufValue *v = value_at(g, i);
    return v && v->type == GV_ARR ? v->etype : -1;
}
extern "C" int64_t ubd_gguf_arr_n(const ubd_gguf *g, int64_t i) {
    const GgufValue *v = value_at(g, i);
    return v && v->type == GV_ARR ? (int64_t)v->n : -1;
}
extern "C" int32_t ubd_gguf_get_int(const ubd_gguf *g, int64_t i, int64_t j, int64_t *out) {
    const GgufValue *v = value_at(g, i);
    if (!elem_ok(v, j) || !out) return UBD_INVALID;
    const int32_t t = v->type == GV_ARR ? v->etype : v->type;
    if (t == GV_STR || t == GV_F32 || t == GV_F64) return UBD_INVALID;
    *out = v->i[(size_t)(j < 0 ? 0 : j)];
    return UBD_OK;
}
extern "C" int32_t ubd_gguf_get_float(const ubd_gguf *g, int64_t i, int64_t j, double *out) {
    const GgufValue *v = value_at(g, i);
    if (!elem_ok(v, j) || !out) return UBD_INVALID;
    const int32_t t = v->type == GV_ARR ? v->etype : v->type;
    if (t != GV_F32 && t != GV_F64) return UBD_INVALID;
    *out = v->f[(size_t)(j < 0 ? 0 : j)];
    return UBD_OK;
}
extern "C" const char *ubd_gguf_get_str(const ubd_gguf *g, int64_t i, int64_t j, uint64_t *len) {
    const GgufValue *v = value_at(g, i);
    if (!elem_ok(v, j)) return nullptr;
    const int32_t t = v->type == GV_ARR ? v->etype : v->type;
    if (t != GV_STR) return nullptr;
    const std::string &s = v->s[(size_t)(j < 0 ? 0 : j)];
    if (len) *len = s.size();
    return s.c_str();
}
extern "C" int64_t ubd_gguf_n_tensors(const ubd_gguf *g) { return g ? (int64_t)g->f.tensors.size() : -1; }
extern "C" int64_t ubd_gguf_find_tensor(const ubd_gguf *g, const char *name) {
    if (!g || !name) return -1;
    auto it = g->f.tensor_index.find(name);
    return it == g->f.tensor_index.end() ? -1 : it->second;
}
extern "C" const char *ubd_gguf_tensor_name(const ubd_gguf *g, int64_t i) {
    const GgufTensor *t = tensor_at(g, i);
    return t ? t->name.c_str() : nullptr;
}
extern "C" int32_t ubd_gguf_tensor_type(const ubd_gguf *g, int64_t i) {
    const GgufTensor *t = tensor_at(g, i);
    return t ? t->type : -1;
}
extern "C" int32_t ubd_gguf_tensor_dims(const ubd_gguf *g, int64_t i, int64_t *ne) {
    const GgufTensor *t = tensor_at(g, i);
    if (!t) return -1;
    if (ne)
        for (int d = 0; d < 4; ++d) ne[d] = t->ne[d];
    return t->n_dims;
}
extern "C" int64_t ubd_gguf_tensor_offset(const ubd_gguf *g, int64_t i) {
    const GgufTensor *t = tensor_at(g, i);
    return t ? (int64_t)(g->f.data_start + t->offset) : -1;
}
extern "C" int64_t ubd_gguf_tensor_nbytes(const ubd_gguf *g, int64_t i) {
    const GgufTensor *t = tensor_at(g, i);
    return t ? (int64_t)t->nbytes : -1;
}

extern "C" int32_t ubd_gguf_model_info(const char *path, ubd_gguf_info *info) {
    if (!path || !info) return UBD_INVALID;
    GgufModel m;
    std::string err;
    if (!open_model(path, &m, &err)) {
        set_error(err);
        return UBD_INVALID;
    }
    info_of(m, info);
    return UBD_OK;
}

extern "C" ubd_model *ubd_model_load_gguf(const char *path, const ubd_model_params *params, int32_t use_mmap,
                                          int32_t *status) {
    auto fail = [&](int32_t code, const std::string &msg) -> ubd_model * {
        set_error("ubd_model_load_gguf: " + msg);
        if (status) *status = code;
        return nullptr;
    };
    if (!path) return fail(UBD_INVALID, "no path");
    GgufModel m;
    std::string err;
    if (!open_model(path, &m, &err)) return fail(UBD_INVALID, err);
    ubd_gguf_info info{};
    info_of(m, &info);
    // the architecture page's Example 8 summary lines
    log_msg(1, "file format = GGUF V%u", info.version);
    log_msg(1, "file type   = %s %s", info.all_same ? "all" : "mostly", gguf_type_name(info.file_type));
    log_msg(1, "file size   = %.2f MiB (%.2f BPW)", info.file_bytes / 1048576.0, info.bpw);
    log_msg(1, "n_layer %d, n_embd %d, n_head %d, n_head_kv %d, n_ff %d, n_vocab %d, model params = %.2f M",
            m.hp.n_layer, m.hp.n_embd, m.hp.n_head, m.hp.n_head_kv, m.hp.n_ff, m.hp.n_vocab, info.n_params / 1e6);

    std::vector<ubd_tensor_src> src;
    std::vector<std::vector<uint8_t>> owned;      // read mode: host copies
    for (auto &kv : m.where) {
        const GgufFile *f = kv.second.first;
        const GgufTensor &t = *kv.second.second;
        ubd_tensor_src s{};
        s.name = t.name.c_str();
        switch (t.type) {
        case GT_F32: s.type = UBD_TYPE_F32; break;
        case GT_F16: s.type = UBD_TYPE_F16; break;
        case GT_BF16: s.type = UBD_TYPE_BF16; break;
        case GT_Q8_0: s.type = UBD_TYPE_Q8_0; break;       // 34-byte blocks: scales stay NULL
        default: return fail(UBD_INVALID, "tensor " + t.name + ": unsupported type");
        }
        if (t.n_dims > 2 || (t.n_dims == 2 && t.ne[1] <= 0)) return fail(UBD_INVALID, "tensor " + t.name + ": not 1-D or 2-D");
        s.ne[0] = t.ne[0];
        s.ne[1] = t.n_dims == 2 ? t.ne[1] : 1;
        if (use_mmap) {
            const uint8_t *base = const_cast<GgufFile *>(f)->map(&err);
            if (!base) return fail(UBD_ALLOC_FAILED, err);
            s.data = base + f->data_start + t.offset;
        } else {
            owned.emplace_back((size_t)t.nbytes);
            if (!f->read(t, owned.back().data(), &err)) return fail(UBD_ALLOC_FAILED, err);
            s.data = owned.back().data();
        }
        src.push_back(s);
    }
    int32_t st = 0;
    ubd_model *model = ubd_model_load(&m.hp, src.data(), (int32_t)src.size(), params, &st);
    if (status) *status = st;
    return model;
}
