"""The binding's filter-spectrum cache (no GPU): a second call at the same grid size builds nothing, an
in-place parameter update or another grid size builds again, and the oldest entry goes first."""
import torch

from attention_free_long_implicit_amd import _lib


def _params(D=4, seed=0):
    g = torch.Generator().manual_seed(seed)
    return {"W1": torch.randn(64, 64, generator=g), "b1": torch.zeros(64), "W2": torch.randn(D, 64, generator=g),
            "b2": torch.zeros(D), "alpha": torch.rand(D, generator=g)}


def test_second_call_at_the_same_length_builds_nothing():
    built = []
    cache = _lib.SpectrumCache(builder=lambda p, shape, mode: built.append((shape, mode)) or ("spectrum", shape))
    ps = [_params(seed=1), _params(seed=2)]
    a = [cache.get(p, (8192,)) for p in ps]
    b = [cache.get(p, (8192,)) for p in ps]
    assert len(built) == 2 and cache.builds == 2
    assert all(x is y for x, y in zip(a, b))
    cache.get(ps[0], (16384,))                      # another length: a new spectrum
    assert len(built) == 3 and built[-1] == ((16384,), _lib.CAUSAL)
    cache.get(ps[0], (8192,), mode=_lib.CIRCULAR)   # another mode
    assert len(built) == 4


def test_in_place_update_of_a_parameter_builds_again():
    built = []
    cache = _lib.SpectrumCache(builder=lambda p, shape, mode: built.append(1) or object())
    p = _params()
    s1 = cache.get(p, (4096,))
    p["alpha"].mul_(2.0)                            # in-place change: version counter moves
    s2 = cache.get(p, (4096,))
    assert len(built) == 2 and s1 is not s2
    assert cache.get(p, (4096,)) is s2 and len(built) == 2


def test_least_recently_used_entry_is_dropped():
    cache = _lib.SpectrumCache(max_entries=2, builder=lambda p, shape, mode: object())
    p = _params()
    a = cache.get(p, (1024,))
    cache.get(p, (2048,))
    cache.get(p, (1024,))                           # 1024 is now the most recent
    cache.get(p, (4096,))                           # drops 2048
    assert cache.get(p, (1024,)) is a and cache.builds == 3
    cache.get(p, (2048,))
    assert cache.builds == 4


def test_operator_from_parameters_uses_the_cache(monkeypatch):
    calls = []
    monkeypatch.setattr(_lib, "operator", lambda v, xs, spectra, y=None, mode=None: calls.append(spectra) or "y")
    cache = _lib.SpectrumCache(builder=lambda p, shape, mode: ("sp", id(p), shape))
    v = torch.zeros(1, 4, 2048)
    xs = [torch.zeros(1, 4, 2048)] * 2
    ps = [_params(seed=3), _params(seed=4)]
    assert _lib.hyena(v, xs, ps, cache=cache) == "y"
    _lib.hyena(v, xs, ps, cache=cache)
    assert cache.builds == 2 and calls[0] == calls[1]
