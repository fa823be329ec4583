"""GPU: a decode cache that grows (prefix fill, appends, per-sequence lengths) against the
CPU oracle's decode over the same cache contents (reading R20: appended K rows are
quantized against the mean of the filled tokens).

Bit-exact checks: appending tokens the cache already holds, into their own slots,
leaves every byte of the cache as the fill wrote it (the append applies the fill's
rules in the fill's layout); appends whose slots lie outside the capacity change
nothing; a decode over lens[b] = S for every sequence equals the plain decode.  The
outputs of grown caches must satisfy max|o - O| <= 2e-3 and ||o - O||_2 / ||O||_2 <=
1e-3 against the unrounded fp64 oracle; a sequence with no token gives zeros.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import int8_w8a8_flashattention_amd as i8

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
REL_L2 = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def i32(a):
    return torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")


def check_close(o16, ref, what):
    o = o16.astype(np.float64)
    err = np.abs(o - ref)
    mx = float(err.max())
    rel = float(np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-30))
    say(f"  {what}: max_abs={mx:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(o)), what
    assert mx <= MAX_ABS, (what, mx)
    assert rel <= REL_L2, (what, rel)


def kv(seed, B, Hkv, S, D):
    g = np.random.Generator(np.random.PCG64(seed))
    off = g.uniform(-3.0, 3.0, (1, 1, 1, D))
    k = (g.standard_normal((B, Hkv, S, D)) + off).astype(np.float16)
    v = g.standard_normal((B, Hkv, S, D)).astype(np.float16)
    return g, k, v


@pytest.mark.parametrize("v_format", ["int8", "fp16"])
@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_append_of_held_tokens_leaves_the_cache_bytes_unchanged(D, v_format):
    B, Hq, Hkv, S, n = 2, 6, 3, 157, 45
    say(f"append into own slots: D={D} {v_format} B={B} Hkv={Hkv} S={S} n={n}")
    g, k, v = kv(800 + D, B, Hkv, S, D)
    nbytes = i8.attn_int8_kvcache_bytes(B, Hkv, S, D, v_format)
    zeros = lambda: torch.zeros(nbytes, dtype=torch.uint8, device="cuda")  # noqa: E731
    a = i8.attn_int8_kvcache_fill(dev(k), dev(v), v_format, cache=zeros())
    b = i8.attn_int8_kvcache_fill(dev(k), dev(v), v_format, cache=zeros())
    ref = host(a.buf).copy()
    assert np.array_equal(host(b.buf), ref)
    tail = slice(S - n, S)
    i8.attn_int8_kvcache_append(b, dev(k[:, :, tail]), dev(v[:, :, tail]), i32([S - n] * B))
    assert np.array_equal(host(b.buf), ref)
    # slots past the capacity, or before slot 0, are not written
    i8.attn_int8_kvcache_append(b, dev(k[:, :, :n]), dev(v[:, :, :n]), i32([S, -n]))
    assert np.array_equal(host(b.buf), ref)
    # two tokens appended into each other's slots: the cache then decodes exactly like
    # the fill of the sequence with those two tokens swapped (the same tokens, so the
    # same exact K mean)
    perm = np.arange(S)
    perm[[10, 140]] = perm[[140, 10]]
    c = i8.attn_int8_kvcache_fill(dev(k[:, :, perm]), dev(v[:, :, perm]), v_format)
    i8.attn_int8_kvcache_append(b, dev(k[:, :, [140]]), dev(v[:, :, [140]]), i32([10] * B))
    i8.attn_int8_kvcache_append(b, dev(k[:, :, [10]]), dev(v[:, :, [10]]), i32([140] * B))
    q = dev(g.standard_normal((B, Hq, D)).astype(np.float16))
    ob, oc = host(i8.attn_int8_decode(q, b)), host(i8.attn_int8_decode(q, c))
    assert np.array_equal(ob.view(np.uint16), oc.view(np.uint16))


@pytest.mark.parametrize("v_format", ["int8", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_lens_of_full_length_equals_decode(D, v_format):
    say(f"decode_lens(S) == decode: D={D} {v_format}")
    B, Hq, Hkv, S = 3, 8, 2, 1500
    g, k, v = kv(810 + D, B, Hkv, S, D)
    q = g.standard_normal((B, Hq, D)).astype(np.float16)
    cache = i8.attn_int8_kvcache_fill(dev(k), dev(v), v_format)
    a = host(i8.attn_int8_decode(dev(q), cache))
    b = host(i8.attn_int8_decode_lens(dev(q), cache, i32([S] * B)))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    # lengths past S are clamped to S, negative ones to 0 (a zero row)
    c = host(i8.attn_int8_decode_lens(dev(q), cache, i32([S + 7, -3, S])))
    assert np.array_equal(c[0].view(np.uint16), a[0].view(np.uint16))
    assert not c[1].any()
    assert np.array_equal(c[2].view(np.uint16), a[2].view(np.uint16))


# (B, Hq, Hkv, S capacity, D, n_fill)
GROW = [
    (2, 4, 2, 200, 32, 37),
    (3, 8, 2, 700, 128, 300),
    (2, 6, 1, 2100, 64, 1),
    (1, 8, 8, 90, 256, 64),
]


@pytest.mark.parametrize("v_format", ["int8", "fp16"])
@pytest.mark.parametrize("shape", GROW, ids=lambda s: "x".join(map(str, s)))
def test_grown_cache_decode_against_oracle(shape, v_format):
    B, Hq, Hkv, S, D, n_fill = shape
    say(f"grown cache: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} n_fill={n_fill} {v_format}")
    g, k, v = kv(820 + D + S, B, Hkv, S, D)
    cache = i8.attn_int8_kvcache_fill_prefix(dev(k[:, :, :n_fill]), dev(v[:, :, :n_fill]), S,
                                             v_format)
    # Every sequence starts with the filled tokens; a step appends to the active ones only
    # (the others get a slot past the capacity, so nothing of theirs is written), so the
    # sequences' lengths, and the slots one append writes, differ between sequences.
    cur = np.full(B, n_fill, dtype=np.int64)
    kf, vf = k.copy(), v.copy()  # the cache's contents slot by slot

    def append(n, active):
        kn = g.standard_normal((B, Hkv, n, D)).astype(np.float16) + k[:, :, :1]
        vn = g.standard_normal((B, Hkv, n, D)).astype(np.float16)
        pos = np.where(active, cur, S)
        i8.attn_int8_kvcache_append(cache, dev(kn), dev(vn), i32(pos))
        for b in np.flatnonzero(active):
            m = min(n, S - cur[b])
            kf[b, :, cur[b]:cur[b] + m] = kn[b, :, :m]
            vf[b, :, cur[b]:cur[b] + m] = vn[b, :, :m]
            cur[b] += m

    def check(what, lens=None):
        lens = cur.copy() if lens is None else np.asarray(lens)
        q = g.standard_normal((B, Hq, D)).astype(np.float16)
        out = host(i8.attn_int8_decode_lens(dev(q), cache, i32(lens)))
        ref = oracle.attn_int8_decode_cache(q, kf, vf, n_fill, lens, v_format=v_format)
        for b in np.flatnonzero(lens == 0):
            assert not out[b].any(), what
        live = lens > 0
        if live.any():
            check_close(out[live], ref[live], f"{what} lens={lens.tolist()}")

    every = np.ones(B, dtype=bool)
    first = np.arange(B) == 0
    check("after the fill")
    append(1, every)
    check("after a one-token append to every sequence")
    append(1, first)
    append(1, ~first)
    append(1, first)
    check("after one-token appends to some sequences")
    shorter = np.maximum(cur - 7 * np.arange(B), 0) * (np.arange(B) != B - 1)
    check("a shorter prefix, and no token", lens=shorter)
    append(41, ~first if B > 1 else every)
    check("after a 41-token append")
    append(S, every)  # fills every sequence up to the capacity; the rest is not written
    assert (cur == S).all()
    check("at capacity")


def test_grown_cache_serving_shape_sampled():
    # the batched serving shape, filled to 8000 of 8192 slots and grown by one token;
    # three sequences are checked against the oracle
    B, Hq, Hkv, S, D, n_fill = 16, 32, 8, 8192, 128, 8000
    say("grown cache at the serving shape")
    g, k, v = kv(830, B, Hkv, S, D)
    for vfmt in ("int8", "fp16"):
        cache = i8.attn_int8_kvcache_fill_prefix(dev(k[:, :, :n_fill]), dev(v[:, :, :n_fill]),
                                                 S, vfmt)
        i8.attn_int8_kvcache_append(cache, dev(k[:, :, n_fill:n_fill + 1]),
                                    dev(v[:, :, n_fill:n_fill + 1]), i32([n_fill] * B))
        lens = np.full(B, n_fill + 1)
        q = g.standard_normal((B, Hq, D)).astype(np.float16)
        out = host(i8.attn_int8_decode_lens(dev(q), cache, i32(lens)))
        for b in (0, 9, 15):
            ref = oracle.attn_int8_decode_cache(q[b:b + 1], k[b:b + 1], v[b:b + 1], n_fill,
                                                lens[b:b + 1], v_format=vfmt)
            check_close(out[b:b + 1], ref, f"{vfmt} sequence {b}")
