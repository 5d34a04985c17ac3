"""ubd_greedy_rows_static, the allocation-free greedy pick, through the C
ABI: its ids equal those of ubd_sample_greedy_all (the context's own greedy
pick, whose workspace the library allocates) on the same logits rows, over
two calls in a row, the second with fewer rows; on planted ties it takes the
lowest index, as NumPy's argmax does; arguments out of range are refused
before anything is enqueued."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model
    from workloads import WORKLOADS, gen_tensor, tensor_specs
    shape = WORKLOADS[1].model
    tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
    return shape, Model(shape, tens, device=0)


def test_static_greedy_equals_the_context_greedy(tiny):
    import torch
    from llama_decode_ubatch_amd import Context, binding
    shape, model = tiny
    V = shape.n_vocab
    ctx = Context(model, n_ctx=512, n_batch=512, n_ubatch=512, n_seq_max=1, type_k="f16", type_v="f16")
    stream = torch.cuda.current_stream(0).cuda_stream
    out = torch.full((binding.UBD_GREEDY_STATIC_MAX_ROWS,), -7, dtype=torch.int32, device="cuda:0")
    for n in (12, 5):                      # two calls in a row, the second with fewer rows
        print(f"static greedy: {n} rows of {V}", flush=True)
        toks = np.random.default_rng(n).integers(0, V, n).astype(np.int32)
        ctx.seq_rm(-1, -1, -1)
        assert ctx.decode(toks, logits=np.ones(n)) == 0
        ref = ctx.greedy_all()
        out.fill_(-7)
        assert binding.greedy_rows_static(0, ctx.logits_device_ptr(), V, n, V, out.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got[:n], ref), (got[:n], ref)
        assert (got[n:] == -7).all()
    ctx.free()


def test_static_greedy_ties_and_shapes():
    import torch
    from llama_decode_ubatch_amd import binding
    stream = torch.cuda.current_stream(0).cuda_stream
    rng = np.random.default_rng(3)
    out = torch.full((binding.UBD_GREEDY_STATIC_MAX_ROWS,), -7, dtype=torch.int32, device="cuda:0")
    for rows, n, ld in ((256, 5000, 5004), (3, 100, 100)):
        print(f"static greedy: {rows} rows of {n} (stride {ld}), planted ties", flush=True)
        z = rng.standard_normal((rows, ld)).astype(np.float32)
        for r in range(rows):
            top = z[r, :n].max() + 1.0
            k = rng.integers(1, 4)
            z[r, rng.choice(n, k, replace=False)] = top       # k-way tie for the maximum
        z[0, :n] = 0.0                                          # all equal: index 0
        z[1, n - 1] = 1e30                                      # the last index
        zd = torch.from_numpy(z).to("cuda:0")
        out.fill_(-7)
        assert binding.greedy_rows_static(0, zd.data_ptr(), ld, rows, n, out.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got[:rows], z[:, :n].argmax(axis=1))
        assert (got[rows:] == -7).all()


def test_static_greedy_refuses_out_of_range():
    import torch
    from llama_decode_ubatch_amd import binding
    stream = torch.cuda.current_stream(0).cuda_stream
    z = torch.zeros((binding.UBD_GREEDY_STATIC_MAX_ROWS + 1, 64), dtype=torch.float32, device="cuda:0")
    out = torch.zeros(binding.UBD_GREEDY_STATIC_MAX_ROWS + 1, dtype=torch.int32, device="cuda:0")
    p, o = z.data_ptr(), out.data_ptr()
    M = binding.UBD_GREEDY_STATIC_MAX_ROWS
    assert binding.greedy_rows_static(0, p, 64, M + 1, 64, o, stream) == binding.UBD_INVALID
    assert binding.greedy_rows_static(0, p, 64, -1, 64, o, stream) == binding.UBD_INVALID
    assert binding.greedy_rows_static(0, p, 64, 2, 6, o, stream) == binding.UBD_INVALID       # not a multiple of 4
    assert binding.greedy_rows_static(0, p, 60, 2, 64, o, stream) == binding.UBD_INVALID      # stride < width
    assert binding.greedy_rows_static(0, p + 4, 64, 2, 64, o, stream) == binding.UBD_INVALID  # unaligned rows
    assert binding.greedy_rows_static(0, 0, 64, 2, 64, o, stream) == binding.UBD_INVALID
    assert binding.greedy_rows_static(-1, p, 64, 2, 64, o, stream) == binding.UBD_INVALID
    assert binding.greedy_rows_static(0, p, 64, 0, 64, o, stream) == binding.UBD_OK           # nothing to do
