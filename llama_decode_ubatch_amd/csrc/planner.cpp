// Host-side decode bookkeeping; see planner.h for the pages it follows.
#include "planner.h"

#include <algorithm>
#include <climits>

namespace ubd {

// ------------------------------------------------------------------ cells
void KVCells::init(int32_t n_stream, int32_t n_cells, bool unified, int32_t n_seq_max) {
    n_stream_ = n_stream;
    n_cells_ = n_cells;
    unified_ = unified;
    n_seq_max_ = n_seq_max;
    n_words_ = (n_seq_max + 31) / 32;
    pos_.assign(n_stream, std::vector<int32_t>(n_cells, -1));
    seqw_.assign(n_stream, std::vector<uint32_t>((size_t)n_words_ * n_cells, 0u));
    free_.assign(n_stream, {});
    used_.assign(n_stream, {});
    for (int32_t st = 0; st < n_stream; ++st)
        for (int32_t c = 0; c < n_cells; ++c) free_[st].insert(free_[st].end(), c);
    seq_pos_.assign(n_seq_max, {});
}

bool KVCells::empty_mask(int32_t st, int32_t c) const {
    for (int32_t w = 0; w < n_words_; ++w)
        if (seqw_[st][(size_t)w * n_cells_ + c]) return false;
    return true;
}

void KVCells::set_cell(int32_t st, int32_t c, int32_t p, const uint32_t *mask) {
    pos_[st][c] = p;
    free_[st].erase(c);
    used_[st].insert(c);
    for (int32_t w = 0; w < n_words_; ++w) {
        seqw_[st][(size_t)w * n_cells_ + c] = mask[w];
        for (uint32_t m = mask[w]; m; m &= m - 1) seq_pos_[32 * w + __builtin_ctz(m)][p] += 1;
    }
}

void KVCells::drop_seq(int32_t st, int32_t c, int32_t s) {
    if (!has(st, c, s)) return;
    seqw_[st][(size_t)(s >> 5) * n_cells_ + c] &= ~(1u << (s & 31));
    auto &m = seq_pos_[s];
    auto it = m.find(pos_[st][c]);
    if (it != m.end() && --it->second == 0) m.erase(it);
    if (empty_mask(st, c)) {
        pos_[st][c] = -1;
        used_[st].erase(c);
        free_[st].insert(c);
    }
}

void KVCells::clear_cell(int32_t st, int32_t c) {
    for (int32_t w = 0; w < n_words_; ++w)
        for (uint32_t x = seqw_[st][(size_t)w * n_cells_ + c]; x; x &= x - 1) drop_seq(st, c, 32 * w + __builtin_ctz(x));
}

int32_t KVCells::seq_pos_max(int32_t s) const {
    if (s < 0 || s >= (int32_t)seq_pos_.size() || seq_pos_[s].empty()) return -1;
    return seq_pos_[s].rbegin()->first;
}

int32_t KVCells::seq_pos_min(int32_t s) const {
    if (s < 0 || s >= (int32_t)seq_pos_.size() || seq_pos_[s].empty()) return -1;
    return seq_pos_[s].begin()->first;
}

void KVCells::seq_rm(int32_t s, int32_t p0, int32_t p1, std::vector<uint8_t> *touched) {
    const int32_t lo = p0 < 0 ? 0 : p0;
    const int32_t hi = p1 < 0 ? INT32_MAX : p1;
    for (int32_t st = 0; st < n_stream_; ++st) {
        if (s >= 0 && st != stream_of(s)) continue;
        std::vector<int32_t> victims;
        for (int32_t c : used_[st]) {
            if (s >= 0 && !has(st, c, s)) continue;
            if (pos_[st][c] >= lo && pos_[st][c] < hi) victims.push_back(c);
        }
        for (int32_t c : victims) {
            if (s >= 0)
                drop_seq(st, c, s);
            else
                clear_cell(st, c);
        }
        if (touched && !victims.empty()) (*touched)[st] = 1;
    }
}

bool KVCells::seq_cp(int32_t src, int32_t dst, int32_t p0, int32_t p1, bool *copied) {
    *copied = false;
    if (src < 0 || dst < 0 || src >= n_seq_max_ || dst >= n_seq_max_) return false;
    if (src == dst) return true;
    const int32_t ss = stream_of(src), sd = stream_of(dst);
    if (ss == sd) {
        const int32_t lo = p0 < 0 ? 0 : p0;
        const int32_t hi = p1 < 0 ? INT32_MAX : p1;
        for (int32_t c : used_[ss]) {
            const int32_t p = pos_[ss][c];
            if (has(ss, c, src) && !has(ss, c, dst) && p >= lo && p < hi) {
                seqw_[ss][(size_t)(dst >> 5) * n_cells_ + c] |= 1u << (dst & 31);
                seq_pos_[dst][p] += 1;
            }
        }
        return true;
    }
    if (p0 >= 0 || p1 >= 0) return false;
    std::vector<int32_t> old(used_[sd].begin(), used_[sd].end());
    for (int32_t c : old) clear_cell(sd, c);
    std::vector<uint32_t> mask(n_words_, 0u);
    mask[dst >> 5] = 1u << (dst & 31);
    std::vector<int32_t> take;
    for (int32_t c : used_[ss])
        if (has(ss, c, src)) take.push_back(c);
    for (int32_t c : take) set_cell(sd, c, pos_[ss][c], mask.data());
    *copied = true;
    return true;
}

void KVCells::seq_keep(int32_t s) {
    for (int32_t st = 0; st < n_stream_; ++st) {
        std::vector<int32_t> cells(used_[st].begin(), used_[st].end());
        for (int32_t c : cells)
            for (int32_t w = 0; w < n_words_; ++w)
                for (uint32_t x = seqw_[st][(size_t)w * n_cells_ + c]; x; x &= x - 1)
                    if (32 * w + __builtin_ctz(x) != s) drop_seq(st, c, 32 * w + __builtin_ctz(x));
    }
}

void KVCells::defrag_plan(std::vector<std::vector<int32_t>> *src) const {
    src->assign(n_stream_, {});
    for (int32_t st = 0; st < n_stream_; ++st) {
        struct Key {
            int32_t seq, pos, cell;
        };
        std::vector<Key> keys;
        for (int32_t c : used_[st]) {
            int32_t first = 0;
            while (!has(st, c, first)) ++first;
            keys.push_back({first, pos_[st][c], c});
        }
        std::sort(keys.begin(), keys.end(), [](const Key &a, const Key &b) {
            if (a.seq != b.seq) return a.seq < b.seq;
            if (a.pos != b.pos) return a.pos < b.pos;
            return a.cell < b.cell;
        });
        for (const Key &k : keys) (*src)[st].push_back(k.cell);
    }
}

void KVCells::defrag_apply(const std::vector<std::vector<int32_t>> &src) {
    for (int32_t st = 0; st < n_stream_; ++st) {
        const auto &order = src[st];
        std::vector<int32_t> pos(order.size());
        std::vector<uint32_t> words((size_t)n_words_ * order.size());
        for (size_t j = 0; j < order.size(); ++j) {
            pos[j] = pos_[st][order[j]];
            for (int32_t w = 0; w < n_words_; ++w)
                words[(size_t)w * order.size() + j] = seqw_[st][(size_t)w * n_cells_ + order[j]];
        }
        std::vector<int32_t> old(used_[st].begin(), used_[st].end());
        for (int32_t c : old) clear_cell(st, c);
        std::vector<uint32_t> mask(n_words_);
        for (size_t j = 0; j < order.size(); ++j) {
            for (int32_t w = 0; w < n_words_; ++w) mask[w] = words[(size_t)w * order.size() + j];
            set_cell(st, (int32_t)j, pos[j], mask.data());
        }
    }
}

bool KVCells::find_slots(std::vector<UBatch> &ubs) const {
    std::vector<std::set<int32_t>::const_iterator> next(n_stream_);
    for (int32_t st = 0; st < n_stream_; ++st) next[st] = free_[st].begin();
    for (auto &ub : ubs) {
        ub.cell.resize(ub.size());
        ub.stream.resize(ub.size());
        for (int32_t t = 0; t < ub.size(); ++t) {
            const int32_t st = stream_of(ub.seq[t]);
            if (next[st] == free_[st].end()) return false;
            ub.stream[t] = st;
            ub.cell[t] = *next[st]++;
        }
    }
    return true;
}

void KVCells::apply(const UBatch &ub) {
    for (int32_t t = 0; t < ub.size(); ++t)
        set_cell(ub.stream[t], ub.cell[t], ub.pos[t], ub.seqw.data() + (size_t)t * n_words_);
}

int32_t KVCells::n_kv(int32_t stream) const {
    return used_[stream].empty() ? 0 : *used_[stream].rbegin() + 1;
}

bool KVCells::fill_sequence(int32_t s, int32_t n, std::vector<int32_t> *cells) {
    const int32_t st = stream_of(s);
    if (seq_pos_max(s) >= 0 || (int64_t)free_[st].size() < n) return false;
    std::vector<int32_t> take;
    take.reserve(n);
    auto it = free_[st].begin();
    for (int32_t i = 0; i < n; ++i) take.push_back(*it++);
    std::vector<uint32_t> mask(n_words_, 0u);
    mask[s >> 5] = 1u << (s & 31);
    for (int32_t i = 0; i < n; ++i) set_cell(st, take[i], i, mask.data());
    if (cells) *cells = std::move(take);
    return true;
}

// ---------------------------------------------------------------- planner
int32_t Planner::init(uint32_t n_ctx_, uint32_t n_batch_, uint32_t n_ubatch_,
                      uint32_t n_seq_max_, bool unified_, int32_t n_vocab_,
                      std::string *err) {
    n_seq_max = n_seq_max_ == 0 ? 1 : n_seq_max_;
    if (n_seq_max > UBD_MAX_SEQ) {
        if (err) *err = "n_seq_max exceeds UBD_MAX_SEQ";
        return UBD_INVALID;
    }
    if (n_ctx_ == 0 || n_batch_ == 0 || n_vocab_ <= 0) {
        if (err) *err = "n_ctx, n_batch and n_vocab must be positive";
        return UBD_INVALID;
    }
    n_ctx = (n_ctx_ + 255u) / 256u * 256u;          // padded to 256 cells
    unified = unified_;
    n_stream = unified ? 1 : n_seq_max;
    n_cells = n_ctx / n_stream;
    if (n_cells == 0) {
        if (err) *err = "n_ctx too small for n_seq_max streams";
        return UBD_INVALID;
    }
    n_batch = std::min(n_ctx, n_batch_);             // causal model
    n_ubatch = std::min(n_batch, n_ubatch_ ? n_ubatch_ : n_batch);
    n_vocab = n_vocab_;
    cells.init((int32_t)n_stream, (int32_t)n_cells, unified, (int32_t)n_seq_max);
    return UBD_OK;
}

int32_t Planner::sanitize(const ubd_batch &b, Clean *c, std::string *err) const {
    auto bad = [&](const char *m) {
        if (err) *err = m;
        return UBD_INVALID;
    };
    if (b.embd) return bad("embeddings input is not supported");
    if (b.n_tokens <= 0) return bad("n_tokens must be positive");
    if ((uint32_t)b.n_tokens > n_batch) return bad("n_tokens exceeds n_batch");
    if (!b.token) return bad("token array is NULL");
    const int32_t n = b.n_tokens;
    c->token.assign(b.token, b.token + n);
    for (int32_t v : c->token)
        if (v < 0 || v >= n_vocab) return bad("token id out of range");
    const int32_t W = cells.n_seq_words();
    c->seq.assign(n, 0);
    c->seqw.assign((size_t)n * W, 0u);
    for (int32_t i = 0; i < n; ++i) {
        uint32_t *m = c->seqw.data() + (size_t)i * W;
        if (!b.seq_id) {
            m[0] = 1u;
            continue;
        }
        const int32_t k = b.n_seq_id ? b.n_seq_id[i] : 1;
        if (k < 1) return bad("n_seq_id must be at least 1");
        if (k > 1 && n_stream != 1) return bad("a token of several sequences needs a unified KV cache");
        if (!b.seq_id[i]) return bad("seq_id row is NULL");
        for (int32_t j = 0; j < k; ++j) {
            const int32_t s = b.seq_id[i][j];
            if (s < 0 || (uint32_t)s >= n_seq_max) return bad("seq_id out of range");
            if ((m[s >> 5] >> (s & 31)) & 1u) return bad("a sequence listed twice for one token");
            m[s >> 5] |= 1u << (s & 31);
        }
        c->seq[i] = b.seq_id[i][0];
    }
    c->seq_order.clear();
    std::vector<uint8_t> seen(n_seq_max, 0);
    for (int32_t s : c->seq)
        if (!seen[s]) {
            seen[s] = 1;
            c->seq_order.push_back(s);
        }
    auto seqs_of = [&](int32_t i, auto &&fn) {
        const uint32_t *m = c->seqw.data() + (size_t)i * W;
        for (int32_t w = 0; w < W; ++w)
            for (uint32_t x = m[w]; x; x &= x - 1) fn(32 * w + __builtin_ctz(x));
    };
    std::vector<int64_t> next(n_seq_max, 0);
    for (int32_t i = 0; i < n; ++i) seqs_of(i, [&](int32_t s) { next[s] = (int64_t)cells.seq_pos_max(s) + 1; });
    c->pos.resize(n);
    if (!b.pos) {
        // autofill from the first sequence of each token
        std::vector<int64_t> fill = next;
        for (int32_t i = 0; i < n; ++i) {
            const int64_t p = fill[c->seq[i]];
            c->pos[i] = (int32_t)p;
            seqs_of(i, [&](int32_t s) { fill[s] = p + 1; });
        }
    } else {
        for (int32_t i = 0; i < n; ++i) c->pos[i] = b.pos[i];
    }
    std::vector<uint8_t> started(n_seq_max, 0);
    bool ok = true;
    for (int32_t i = 0; i < n && ok; ++i) {
        const int32_t p = c->pos[i];
        seqs_of(i, [&](int32_t s) {
            if (!started[s] && next[s] == 0) {
                // an empty sequence may start at any position >= 0
                if (p < 0) ok = false;
                next[s] = p;
            }
            started[s] = 1;
            if (p != next[s]) ok = false;
            ++next[s];
        });
    }
    if (!ok) return bad("positions must continue each sequence consecutively");
    c->out.assign(n, 0);
    if (!b.logits) {
        c->out[n - 1] = 1;
    } else {
        for (int32_t i = 0; i < n; ++i) c->out[i] = b.logits[i] != 0;
    }
    return UBD_OK;
}

void Planner::push_ubatch(const Clean &c, const std::vector<int32_t> &idx,
                          int32_t n_seq_tokens, int32_t n_seqs) {
    UBatch ub;
    ub.idx = idx;
    ub.n_seq_tokens = n_seq_tokens;
    ub.n_seqs = n_seqs;
    const int32_t W = cells.n_seq_words();
    for (int32_t i : idx) {
        ub.token.push_back(c.token[i]);
        ub.pos.push_back(c.pos[i]);
        ub.seq.push_back(c.seq[i]);
        ub.seqw.insert(ub.seqw.end(), c.seqw.begin() + (size_t)i * W, c.seqw.begin() + (size_t)(i + 1) * W);
    }
    ubatches.push_back(std::move(ub));
}

void Planner::split_simple(const Clean &c) {
    const int32_t n = (int32_t)c.token.size();
    for (int32_t i = 0; i < n; i += (int32_t)n_ubatch) {
        const int32_t e = std::min<int32_t>(n, i + (int32_t)n_ubatch);
        std::vector<int32_t> idx;
        for (int32_t j = i; j < e; ++j) idx.push_back(j);
        push_ubatch(c, idx, e - i, 1);
    }
}

void Planner::split_equal(const Clean &c) {
    // per-sequence queues in batch order
    std::vector<std::vector<int32_t>> q(n_seq_max);
    for (int32_t i = 0; i < (int32_t)c.token.size(); ++i) q[c.seq[i]].push_back(i);
    std::vector<size_t> head(n_seq_max, 0);
    for (;;) {
        std::vector<int32_t> live;
        for (int32_t s : c.seq_order)
            if (head[s] < q[s].size() && live.size() < n_ubatch) live.push_back(s);
        if (live.empty()) return;
        size_t k = n_ubatch / live.size();
        for (int32_t s : live) k = std::min(k, q[s].size() - head[s]);
        std::vector<int32_t> idx;
        for (int32_t s : live) {
            for (size_t j = 0; j < k; ++j) idx.push_back(q[s][head[s] + j]);
            head[s] += k;
        }
        push_ubatch(c, idx, (int32_t)k, (int32_t)live.size());
    }
}

void Planner::rollback(const UBatch &ub, Executor *ex) {
    const int32_t W = cells.n_seq_words();
    std::map<int32_t, int32_t> pos_min;
    for (int32_t t = 0; t < ub.size(); ++t)
        for (int32_t w = 0; w < W; ++w)
            for (uint32_t x = ub.seqw[(size_t)t * W + w]; x; x &= x - 1) {
                const int32_t s = 32 * w + __builtin_ctz(x);
                auto it = pos_min.find(s);
                if (it == pos_min.end() || ub.pos[t] < it->second) pos_min[s] = ub.pos[t];
            }
    std::vector<uint8_t> touched(n_stream, 0);
    for (auto &kv : pos_min) cells.seq_rm(kv.first, kv.second, -1, &touched);
    if (ex) ex->cells_changed(touched);
}

bool Planner::seq_rm(int32_t s, int32_t p0, int32_t p1, Executor *ex) {
    if (s >= (int32_t)n_seq_max) return false;
    std::vector<uint8_t> touched(n_stream, 0);
    cells.seq_rm(s, p0, p1, &touched);
    if (ex) ex->cells_changed(touched);
    return true;
}

bool Planner::seq_cp(int32_t src, int32_t dst, int32_t p0, int32_t p1, Executor *ex) {
    if (src < 0 || dst < 0 || src >= (int32_t)n_seq_max || dst >= (int32_t)n_seq_max) return false;
    if (src == dst) return true;
    const int32_t ss = cells.stream_of(src), sd = cells.stream_of(dst);
    if (ss != sd) {
        if (p0 >= 0 || p1 >= 0) return false;
        if (ex && ex->stream_copy(ss, sd) != UBD_OK) return false;
    }
    bool copied = false;
    if (!cells.seq_cp(src, dst, p0, p1, &copied)) return false;
    std::vector<uint8_t> touched(n_stream, 0);
    touched[sd] = 1;
    if (ex) ex->cells_changed(touched);
    return true;
}

bool Planner::seq_keep(int32_t s, Executor *ex) {
    if (s < 0 || s >= (int32_t)n_seq_max) return false;
    cells.seq_keep(s);
    std::vector<uint8_t> touched(n_stream, 1);
    if (ex) ex->cells_changed(touched);
    return true;
}

int32_t Planner::defrag(Executor *ex) {
    std::vector<std::vector<int32_t>> src;
    cells.defrag_plan(&src);
    int32_t moved = 0;
    std::vector<uint8_t> touched(n_stream, 0);
    for (uint32_t st = 0; st < n_stream; ++st)
        for (size_t j = 0; j < src[st].size(); ++j)
            if (src[st][j] != (int32_t)j) {
                ++moved;
                touched[st] = 1;
            }
    if (moved == 0) return 0;
    if (ex) {
        const int32_t rc = ex->cells_move(src);
        if (rc != UBD_OK) return rc;
    }
    cells.defrag_apply(src);
    if (ex) ex->cells_changed(touched);
    return moved;
}

int32_t Planner::decode(const ubd_batch &b, Executor *ex, std::string *err) {
    ubatches.clear();
    out_row.clear();
    cell_of.clear();
    n_outputs = 0;
    last_ok = false;
    Clean c;
    int32_t rc = sanitize(b, &c, err);
    if (rc != UBD_OK) return rc;
    if (n_stream == 1)
        split_simple(c);
    else
        split_equal(c);
    // The decode-loop page ("KV cache details") compacts the cache and
    // searches again after a failed search.  This search takes any free cell
    // of the stream and compaction keeps the count of free cells, so that
    // second search cannot succeed: return at once, nothing changed.
    if (!cells.find_slots(ubatches)) {
        if (err) *err = "no KV slot for the batch";
        ubatches.clear();
        return UBD_NO_KV_SLOT;
    }
    const int32_t n = b.n_tokens;
    out_row.assign(n, -1);
    for (int32_t i = 0; i < n; ++i)
        if (c.out[i]) out_row[i] = n_outputs++;
    if (ex) {
        rc = ex->reserve_outputs(n_outputs);
        if (rc != UBD_OK) {
            if (err && err->empty()) *err = "cannot reserve the output buffer";
            ubatches.clear();
            return rc;
        }
    }
    cell_of.assign(n, -1);
    for (auto &ub : ubatches) {
        ub.out_row.resize(ub.size());
        ub.n_outputs = 0;
        for (int32_t t = 0; t < ub.size(); ++t) {
            ub.out_row[t] = out_row[ub.idx[t]];
            ub.n_outputs += ub.out_row[t] >= 0;
            cell_of[ub.idx[t]] = ub.cell[t];
        }
    }
    for (int32_t k = 0; k < (int32_t)ubatches.size(); ++k) {
        const UBatch &ub = ubatches[k];
        cells.apply(ub);                       // commit before compute
        rc = ex ? ex->run_ubatch(ub, k) : UBD_OK;
        if (rc != UBD_OK) {
            rollback(ub, ex);
            if (err && err->empty()) *err = "ubatch failed";
            return rc;
        }
    }
    last_ok = true;
    return UBD_OK;
}

}  // namespace ubd
