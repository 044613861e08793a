"""GPU checks at the largest row the library accepts (n = 2^32 - 2, indices
up to 2^32 - 3, composite index field of 32 bits, 8-16 GB rows).  The CPU
oracle cannot hold these rows, so the answers are checked through properties
that hold at any size (every output is the input element at its index, the
order is value descending then index ascending, nothing outside the output
outranks its last element) or against a closed form (planted values over a
constant row)."""
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_MAX = 2 ** 32 - 2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tss():
    import top_selection_sample_amd as tss
    return tss


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _first_true(mask, m, chunk=2 ** 30):
    """Indices of the first m true entries (torch's nonzero is taken per
    chunk: it does not handle 2^32 entries in one call)."""
    out, got = [], 0
    for s in range(0, mask.numel(), chunk):
        nz = torch.nonzero(mask[s:s + chunk]).flatten() + s
        out.append(nz[: m - got])
        got += out[-1].numel()
        if got >= m:
            break
    return torch.cat(out)


def _check_by_properties(x, v, i, k):
    """x: 1-D input without NaN; v, i: the k outputs."""
    assert v.shape == (k,) and i.shape == (k,)
    assert int(i.min()) >= 0 and int(i.max()) < x.numel()
    assert torch.equal(_bits(x[i]), _bits(v)), "values are not the input's bits"
    assert torch.unique(i).numel() == k, "repeated index"
    vf = v.float()
    assert bool((vf[1:] <= vf[:-1]).all()), "values not in descending order"
    eq = vf[1:] == vf[:-1]
    assert bool((i[1:][eq] > i[:-1][eq]).all()), "equal values not in index order"
    vk = v[-1]
    assert int((x > vk).sum()) == int((v > vk).sum()), "an element above the last output is missing"
    m = int((v == vk).sum())
    ties = _first_true(x == vk, m)
    assert torch.equal(ties, i[v == vk]), "ties of the last output are not the lowest indices"


def test_max_row_fp32_normal_with_planted_high_indices():
    tss = _tss()
    g = torch.Generator(device="cuda").manual_seed(4242)
    say(f"max row: fp32 n={N_MAX} standard normal, three planted maxima at high indices")
    x = torch.randn(N_MAX, device="cuda", generator=g)
    pos = torch.tensor([N_MAX - 1, 2 ** 31 + 5, 2 ** 32 - 100], device="cuda")
    x[pos] = torch.tensor([1e30, 1e29, 1e28], device="cuda")
    for k in (64, 20_000):
        say(f"  k={k}")
        v, i = tss.topk(x, k)
        torch.cuda.synchronize()
        assert i[:3].tolist() == pos.tolist()
        _check_by_properties(x, v, i, k)
        st = tss.read_stats(1)[0]
        assert st["path"] in (0, 1) and st["flags"] == 0
    del x, v, i
    torch.cuda.empty_cache()


@pytest.mark.parametrize("route", ["auto", "exact"])
def test_max_row_bf16_constant_with_planted(route):
    # zeros with ten planted values: the answer is the planted values (largest
    # first), then the lowest-index zeros; the zeros tie far beyond any buffer,
    # so the index digits of the composite decide (bits 31..0 of the index)
    tss = _tss()
    k = 64
    say(f"max row: bf16 n={N_MAX} zeros + 10 planted, k={k}, route {route}")
    x = torch.zeros(N_MAX, dtype=torch.bfloat16, device="cuda")
    pos = [5, 2 ** 31 - 1, 2 ** 31, 2 ** 31 + 1, 3_000_000_000, N_MAX - 1, 17, 2 ** 32 - 200,
           1_000_000, 4_000_000_000]
    vals = [float(j + 1) for j in range(10)]          # exact in bf16
    x[torch.tensor(pos, device="cuda")] = torch.tensor(vals, device="cuda").to(torch.bfloat16)
    params = tss.default_params(force_path=tss.PATH_EXACT) if route == "exact" else None
    v, i = tss.topk(x, k, params=params)
    torch.cuda.synchronize()
    order = sorted(range(10), key=lambda j: -vals[j])
    zeros = [j for j in range(k + 10) if j not in pos][: k - 10]
    assert i.tolist() == [pos[j] for j in order] + zeros
    assert v.float().tolist() == [vals[j] for j in order] + [0.0] * (k - 10)
    assert bool((_bits(v[10:]) == 0).all())   # +0.0 bits
    st = tss.read_stats(1)[0]
    assert st["flags"] == 0
    assert st["path"] == (2 if route == "exact" else 1)
    del x, v, i
    torch.cuda.empty_cache()
