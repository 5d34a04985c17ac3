// Host-side bookkeeping of one decode call: batch validation and autofill,
// ubatch splitting, KV-cell slot search / commit / removal and the decode
// control flow with its return codes.  Pure C++ (no HIP): the GPU context
// plugs its forward pass in through Executor, the host-only planner entry
// points use a stub.
//
// Pages: "llama.cpp AI LLM Engine - how it works", Steps 10-12 (batch fields,
// tokens of several sequences, allocator autofill and checks, init_batch
// splitting and all-or-nothing slot preparation, return codes); "Decode
// loop: batching, KV cache, memory management", sections "Batch pipeline",
// "KV cache details" (cells with a position and a shareable set of
// sequences; defrag, also as the retry of a failed slot search) and "Error
// recovery and state rollback".
#pragma once

#include <cstdint>
#include <map>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "ubd.h"

namespace ubd {

struct UBatch {
    std::vector<int32_t> idx;      // batch index of each token (ubatch order)
    std::vector<int32_t> token;
    std::vector<int32_t> pos;
    std::vector<int32_t> seq;      // first sequence of each token
    std::vector<uint32_t> seqw;    // [token][n_seq_words] all its sequences
    std::vector<int32_t> stream;   // KV stream of the token's sequence
    std::vector<int32_t> cell;     // KV cell within the stream
    std::vector<int32_t> out_row;  // output row or -1
    int32_t n_seq_tokens = 0;
    int32_t n_seqs = 0;
    int32_t n_outputs = 0;
    int32_t size() const { return (int32_t)idx.size(); }
};

// Per-stream cell tables.  A cell holds a position (-1 = empty) and the set
// of sequences using it as n_seq_words 32-bit words, word w of all cells of
// a stream stored together (the layout the attention kernels read).  A cell
// with no sequence left is empty.
class KVCells {
public:
    void init(int32_t n_stream, int32_t n_cells, bool unified, int32_t n_seq_max);
    int32_t stream_of(int32_t s) const { return unified_ ? 0 : s; }
    int32_t n_stream() const { return n_stream_; }
    int32_t n_cells() const { return n_cells_; }
    int32_t n_seq_words() const { return n_words_; }
    int32_t seq_pos_max(int32_t s) const;
    int32_t seq_pos_min(int32_t s) const;
    // Takes s (every sequence if s < 0) out of the cells with p0 <= pos <
    // p1; marks the streams it changed.
    void seq_rm(int32_t s, int32_t p0, int32_t p1, std::vector<uint8_t> *touched);
    // Adds dst to src's cells in range (same stream), or makes dst's stream
    // a copy of src's with dst in place of src (whole range only; *copied
    // set).  False for invalid arguments.
    bool seq_cp(int32_t src, int32_t dst, int32_t p0, int32_t p1, bool *copied);
    void seq_keep(int32_t s);
    // Compaction plan: per stream, src[j] = the cell that moves to j, for
    // the occupied cells ordered by (lowest sequence, position, index).
    void defrag_plan(std::vector<std::vector<int32_t>> *src) const;
    void defrag_apply(const std::vector<std::vector<int32_t>> &src);
    // Lowest empty cell of its stream for every token, ubatch after ubatch,
    // without committing anything.  False if some token finds none.
    bool find_slots(std::vector<UBatch> &ubs) const;
    void apply(const UBatch &ub);
    // Cells an attention pass has to scan in a stream: highest used + 1.
    int32_t n_kv(int32_t stream) const;
    int32_t n_used(int32_t stream) const { return (int32_t)used_[stream].size(); }
    // Occupy the n lowest empty cells of s's stream with positions 0..n-1.
    bool fill_sequence(int32_t s, int32_t n, std::vector<int32_t> *cells);
    int32_t pos_at(int32_t st, int32_t c) const { return pos_[st][c]; }
    bool has(int32_t st, int32_t c, int32_t s) const {
        return (seqw_[st][(size_t)(s >> 5) * n_cells_ + c] >> (s & 31)) & 1u;
    }
    const int32_t *pos_data(int32_t st) const { return pos_[st].data(); }
    const uint32_t *seq_words(int32_t st) const { return seqw_[st].data(); }

private:
    void set_cell(int32_t st, int32_t c, int32_t p, const uint32_t *mask);
    void drop_seq(int32_t st, int32_t c, int32_t s);
    void clear_cell(int32_t st, int32_t c);
    bool empty_mask(int32_t st, int32_t c) const;

    int32_t n_stream_ = 0, n_cells_ = 0, n_words_ = 1, n_seq_max_ = 1;
    bool unified_ = false;
    std::vector<std::vector<int32_t>> pos_;
    std::vector<std::vector<uint32_t>> seqw_;
    std::vector<std::set<int32_t>> free_, used_;
    std::vector<std::map<int32_t, int32_t>> seq_pos_;   // per sequence: pos -> cells
};

// The GPU context implements this; run_ubatch enqueues one forward pass
// after the ubatch's cells were committed and returns UBD_OK,
// UBD_ABORTED, UBD_ALLOC_FAILED or UBD_COMPUTE_FAILED.  The memory hooks
// mirror cell-table changes and move K/V rows; they return UBD_OK or an
// error code.
struct Executor {
    virtual ~Executor() = default;
    virtual int32_t run_ubatch(const UBatch &ub, int32_t k) = 0;
    // Room for n output rows, before any ubatch is committed.
    virtual int32_t reserve_outputs(int32_t n) { (void)n; return UBD_OK; }
    // The tables of the marked streams changed.
    virtual int32_t cells_changed(const std::vector<uint8_t> &touched) { (void)touched; return UBD_OK; }
    // K/V rows of every cell of stream src copied to stream dst (before the
    // tables change).
    virtual int32_t stream_copy(int32_t src, int32_t dst) { (void)src; (void)dst; return UBD_OK; }
    // K/V rows move within each stream: cell j <- cell src[st][j] (before
    // the tables change).
    virtual int32_t cells_move(const std::vector<std::vector<int32_t>> &src) { (void)src; return UBD_OK; }
};

class Planner {
public:
    // Resolved context geometry.  Returns UBD_OK or UBD_INVALID.
    int32_t init(uint32_t n_ctx, uint32_t n_batch, uint32_t n_ubatch,
                 uint32_t n_seq_max, bool unified, int32_t n_vocab,
                 std::string *err);
    int32_t decode(const ubd_batch &b, Executor *ex, std::string *err);
    bool seq_rm(int32_t s, int32_t p0, int32_t p1, Executor *ex);
    bool seq_cp(int32_t src, int32_t dst, int32_t p0, int32_t p1, Executor *ex);
    bool seq_keep(int32_t s, Executor *ex);
    // Compacts every stream; returns the number of cells that moved, or a
    // negative error code of the executor.
    int32_t defrag(Executor *ex);

    uint32_t n_ctx = 0, n_batch = 0, n_ubatch = 0, n_seq_max = 0;
    uint32_t n_stream = 0, n_cells = 0;
    bool unified = false;
    int32_t n_vocab = 0;
    KVCells cells;

    // results of the last decode
    std::vector<UBatch> ubatches;
    std::vector<int32_t> out_row;     // per batch index
    std::vector<int32_t> cell_of;     // per batch index
    int32_t n_outputs = 0;
    bool last_ok = false;

private:
    struct Clean {
        std::vector<int32_t> token, pos, seq;
        std::vector<uint32_t> seqw;       // [token][n_seq_words]
        std::vector<uint8_t> out;
        std::vector<int32_t> seq_order;   // first appearance
    };
    int32_t sanitize(const ubd_batch &b, Clean *c, std::string *err) const;
    void split_simple(const Clean &c);
    void split_equal(const Clean &c);
    void push_ubatch(const Clean &c, const std::vector<int32_t> &idx,
                     int32_t n_seq_tokens, int32_t n_seqs);
    void rollback(const UBatch &ub, Executor *ex);
};

}  // namespace ubd
