// Randomised drive of the host planner (batch sanitising, ubatch splits, KV
// cell search, rollback, sequence operations, defrag) for a build with the
// address and undefined-behaviour sanitizers: every call path runs many
// times on valid and invalid input, and the cell tables are checked against
// their own invariants after every step.  Host code only (no GPU).
//
//   g++ -std=c++17 -O1 -g -fsanitize=address,undefined -fno-omit-frame-pointer \
//       -I include -I llama_decode_ubatch_amd/csrc \
//       tests/planner_sanitize.cpp llama_decode_ubatch_amd/csrc/planner.cpp
#include "planner.h"

#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

using namespace ubd;

namespace {

// Executor that fails a chosen ubatch, to drive the rollback path.
struct FailingExecutor : Executor {
    int fail_at = -1, fail_code = UBD_COMPUTE_FAILED;
    int32_t run_ubatch(const UBatch &ub, int32_t k) override {
        (void)ub;
        return k == fail_at ? fail_code : UBD_OK;
    }
};

int g_failures = 0;
void check(bool ok, const char *what, int iter) {
    if (!ok) {
        std::fprintf(stderr, "invariant failed at step %d: %s\n", iter, what);
        ++g_failures;
    }
}

// Every sequence's positions: min <= max, both -1 or both >= 0; the cells
// in use never exceed the stream size; cells beyond n_kv are empty.
void check_tables(const Planner &P, int iter) {
    for (uint32_t s = 0; s < P.n_seq_max; ++s) {
        const int32_t lo = P.cells.seq_pos_min((int32_t)s), hi = P.cells.seq_pos_max((int32_t)s);
        check((lo < 0) == (hi < 0), "pos_min / pos_max both set or both empty", iter);
        check(lo <= hi, "pos_min <= pos_max", iter);
    }
    for (uint32_t st = 0; st < P.n_stream; ++st) {
        const int32_t nkv = P.cells.n_kv((int32_t)st);
        check(nkv >= 0 && nkv <= (int32_t)P.n_cells, "n_kv within the stream", iter);
        check(P.cells.n_used((int32_t)st) <= nkv, "cells in use below n_kv", iter);
        for (int32_t c = nkv; c < (int32_t)P.n_cells; ++c)
            check(P.cells.pos_at((int32_t)st, c) < 0, "cells past n_kv are empty", iter);
    }
}

}  // namespace

int main(int argc, char **argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 4000;
    std::mt19937 rng(12345);
    auto uni = [&](int a, int b) { return std::uniform_int_distribution<int>(a, b)(rng); };
    const int32_t n_vocab = 1000;
    int runs = 0, n_ok = 0, n_slot = 0, n_inval = 0, n_fail = 0;
    for (int cfg = 0; cfg < 8; ++cfg) {
        const bool unified = cfg & 1;
        const uint32_t n_seq_max = (uint32_t)(cfg & 2 ? 40 : 4);     // 40: two sequence-mask words
        const uint32_t n_ctx = cfg & 4 ? 256 : 1024;
        Planner P;
        std::string err;
        if (P.init(n_ctx, 512, (uint32_t)uni(1, 64), n_seq_max, unified, n_vocab, &err) != UBD_OK) {
            std::fprintf(stderr, "init failed: %s\n", err.c_str());
            return 2;
        }
        FailingExecutor ex;
        for (int it = 0; it < iters; ++it) {
            const int op = uni(0, 9);
            if (op <= 5) {
                // a batch: mostly valid continuations, sometimes broken
                const int n = uni(0, 40);
                std::vector<ubd_token> tok(n);
                std::vector<ubd_pos> pos(n);
                std::vector<int32_t> nsid(n);
                std::vector<ubd_seq_id> sid_store((size_t)n * 3);
                std::vector<ubd_seq_id *> sid(n);
                std::vector<int8_t> lg(n);
                std::vector<int32_t> next(n_seq_max);
                for (uint32_t s = 0; s < n_seq_max; ++s) next[s] = P.cells.seq_pos_max((int32_t)s) + 1;
                for (int i = 0; i < n; ++i) {
                    const int s = uni(0, (int)n_seq_max - 1);
                    tok[i] = uni(0, 20) == 0 ? uni(-5, n_vocab + 5) : uni(0, n_vocab - 1);
                    nsid[i] = uni(0, 15) == 0 ? uni(0, 3) : 1;
                    sid[i] = &sid_store[(size_t)i * 3];
                    for (int j = 0; j < 3; ++j) sid[i][j] = uni(0, 25) == 0 ? uni(-2, (int)n_seq_max + 2) : (s + j) % (int)n_seq_max;
                    pos[i] = uni(0, 25) == 0 ? uni(-3, 2000) : next[s]++;
                    lg[i] = (int8_t)uni(0, 1);
                }
                ubd_batch b{};
                b.n_tokens = n;
                b.token = tok.data();
                const int form = uni(0, 3);               // NULL arrays take the autofill paths
                b.pos = form & 1 ? pos.data() : nullptr;
                b.n_seq_id = form & 2 ? nsid.data() : nullptr;
                b.seq_id = form & 2 ? sid.data() : nullptr;
                b.logits = uni(0, 1) ? lg.data() : nullptr;
                ex.fail_at = uni(0, 6) == 0 ? uni(0, 3) : -1;
                ex.fail_code = uni(0, 1) ? UBD_COMPUTE_FAILED : UBD_ABORTED;
                const int32_t rc = P.decode(b, &ex, &err);
                check(rc == UBD_OK || rc == UBD_NO_KV_SLOT || rc == UBD_INVALID || rc == ex.fail_code,
                      "decode returns a documented code", it);
                n_ok += rc == UBD_OK;
                n_slot += rc == UBD_NO_KV_SLOT;
                n_inval += rc == UBD_INVALID;
                n_fail += rc == ex.fail_code;
                if (rc == UBD_OK) {
                    check((int32_t)P.out_row.size() == n && (int32_t)P.cell_of.size() == n, "per-token results", it);
                    for (int i = 0; i < n; ++i) check(P.cell_of[i] >= 0 && P.cell_of[i] < (int32_t)P.n_cells,
                                                      "assigned cell in range", it);
                }
                ++runs;
            } else if (op == 6) {
                P.seq_rm(uni(-1, (int)n_seq_max), uni(-2, 600), uni(-2, 600), nullptr);
            } else if (op == 7) {
                P.seq_cp(uni(-1, (int)n_seq_max), uni(-1, (int)n_seq_max), uni(-2, 600), uni(-2, 600), nullptr);
            } else if (op == 8) {
                if (uni(0, 5) == 0) P.seq_keep(uni(-1, (int)n_seq_max), nullptr);
            } else {
                const int32_t moved = P.defrag(nullptr);
                check(moved >= 0, "defrag without an executor cannot fail", it);
            }
            check_tables(P, it);
        }
    }
    std::printf("planner drive: %d decode calls (ok %d, no slot %d, invalid %d, rolled back %d), "
                "%d invariant failures\n", runs, n_ok, n_slot, n_inval, n_fail, g_failures);
    // every return path must have been taken
    return g_failures == 0 && n_ok && n_slot && n_inval && n_fail ? 0 : 1;
}
