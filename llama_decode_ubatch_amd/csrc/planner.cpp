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
    pos_.assign(n_stream, std::vector<int32_t>(n_cells, -1));
    seq_.assign(n_stream, std::vector<int32_t>(n_cells, -1));
    free_.assign(n_stream, {});
    used_.assign(n_stream, {});
    for (int32_t st = 0; st < n_stream; ++st)
        for (int32_t c = 0; c < n_cells; ++c) free_[st].insert(free_[st].end(), c);
    seq_pos_.assign(n_seq_max, {});
}

void KVCells::set_cell(int32_t st, int32_t c, int32_t p, int32_t s) {
    pos_[st][c] = p;
    seq_[st][c] = s;
    free_[st].erase(c);
    used_[st].insert(c);
    seq_pos_[s][p] += 1;
}

void KVCells::clear_cell(int32_t st, int32_t c) {
    int32_t s = seq_[st][c], p = pos_[st][c];
    auto &m = seq_pos_[s];
    auto it = m.find(p);
    if (it != m.end() && --it->second == 0) m.erase(it);
    pos_[st][c] = -1;
    seq_[st][c] = -1;
    used_[st].erase(c);
    free_[st].insert(c);
}

int32_t KVCells::seq_pos_max(int32_t s) const {
    if (s < 0 || s >= (int32_t)seq_pos_.size() || seq_pos_[s].empty()) return -1;
    return seq_pos_[s].rbegin()->first;
}

int32_t KVCells::seq_pos_min(int32_t s) const {
    if (s < 0 || s >= (int32_t)seq_pos_.size() || seq_pos_[s].empty()) return -1;
    return seq_pos_[s].begin()->first;
}

void KVCells::seq_rm(int32_t s, int32_t p0, int32_t p1,
                     std::vector<std::pair<int32_t, int32_t>> *cleared) {
    const int32_t lo = p0 < 0 ? 0 : p0;
    const int32_t hi = p1 < 0 ? INT32_MAX : p1;
    for (int32_t st = 0; st < n_stream_; ++st) {
        if (s >= 0 && st != stream_of(s)) continue;
        std::vector<int32_t> victims;
        for (int32_t c : used_[st]) {
            if (s >= 0 && seq_[st][c] != s) continue;
            if (pos_[st][c] >= lo && pos_[st][c] < hi) victims.push_back(c);
        }
        for (int32_t c : victims) {
            clear_cell(st, c);
            if (cleared) cleared->emplace_back(st, c);
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
    for (int32_t t = 0; t < ub.size(); ++t) set_cell(ub.stream[t], ub.cell[t], ub.pos[t], ub.seq[t]);
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
    for (int32_t i = 0; i < n; ++i) set_cell(st, take[i], i, s);
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
    c->seq.assign(n, 0);
    if (b.seq_id) {
        for (int32_t i = 0; i < n; ++i) {
            if (b.n_seq_id && b.n_seq_id[i] != 1) return bad("n_seq_id must be 1");
            if (!b.seq_id[i]) return bad("seq_id row is NULL");
            c->seq[i] = b.seq_id[i][0];
        }
    }
    for (int32_t s : c->seq)
        if (s < 0 || (uint32_t)s >= n_seq_max) return bad("seq_id out of range");
    c->seq_order.clear();
    std::vector<uint8_t> seen(n_seq_max, 0);
    for (int32_t s : c->seq)
        if (!seen[s]) {
            seen[s] = 1;
            c->seq_order.push_back(s);
        }
    std::vector<int64_t> next(n_seq_max, 0);
    for (int32_t s : c->seq_order) next[s] = (int64_t)cells.seq_pos_max(s) + 1;
    c->pos.resize(n);
    if (!b.pos) {
        for (int32_t i = 0; i < n; ++i) c->pos[i] = (int32_t)next[c->seq[i]]++;
    } else {
        std::vector<uint8_t> started(n_seq_max, 0);
        for (int32_t i = 0; i < n; ++i) {
            const int32_t s = c->seq[i];
            const int32_t p = b.pos[i];
            if (!started[s] && next[s] == 0) {
                // an empty sequence may start at any position >= 0
                if (p < 0) return bad("negative position");
                next[s] = p;
            }
            started[s] = 1;
            if (p != next[s]) return bad("positions must continue each sequence consecutively");
            ++next[s];
            c->pos[i] = p;
        }
    }
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
    for (int32_t i : idx) {
        ub.token.push_back(c.token[i]);
        ub.pos.push_back(c.pos[i]);
        ub.seq.push_back(c.seq[i]);
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
    std::map<int32_t, int32_t> pos_min;
    for (int32_t t = 0; t < ub.size(); ++t) {
        auto it = pos_min.find(ub.seq[t]);
        if (it == pos_min.end() || ub.pos[t] < it->second) pos_min[ub.seq[t]] = ub.pos[t];
    }
    std::vector<std::pair<int32_t, int32_t>> cleared;
    for (auto &kv : pos_min) cells.seq_rm(kv.first, kv.second, -1, &cleared);
    if (ex && !cleared.empty()) ex->cells_cleared(cleared);
}

bool Planner::seq_rm(int32_t s, int32_t p0, int32_t p1, Executor *ex) {
    if (s >= (int32_t)n_seq_max) return false;
    std::vector<std::pair<int32_t, int32_t>> cleared;
    cells.seq_rm(s, p0, p1, &cleared);
    if (ex && !cleared.empty()) ex->cells_cleared(cleared);
    return true;
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
