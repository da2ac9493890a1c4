"""GPU parity of wa_encoder_attn against the oracle (max-abs 2e-2, mean-abs 2e-3)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import attn
from tests.gpu_helpers import announce, assert_close, to_dev

pytestmark = pytest.mark.gpu

POISON = float("nan")


def _gpu(wa, q, k, v, lens, causal, views=None):
    qd, kd, vd = views if views is not None else (to_dev(q), to_dev(k), to_dev(v))
    out = torch.full(qd.shape, POISON, dtype=torch.bfloat16, device="cuda")
    ld = None if lens is None else to_dev(np.asarray(lens, np.int32))
    wa.wa_encoder_attn(qd, kd, vd, out=out, lens=ld, causal=causal, softmax_scale=0.125)
    torch.cuda.synchronize()
    return out


def _check(got, q, k, v, lens, causal, what, pairs=None):
    """Compare valid rows; rows at or beyond a length must still hold the poison."""
    B, T, H, _ = q.shape
    lens_a = np.full(B, T) if lens is None else np.asarray(lens)
    g = got.float().cpu().numpy()
    for b in range(B):
        assert np.all(np.isnan(g[b, lens_a[b]:])), f"{what}: rows beyond len {lens_a[b]} of seq {b} written"
    if pairs is None:
        want, mag = attn.dense_attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), lens_a,
                                         causal, 0.125, with_magnitude=True)
        mask = np.arange(T)[None, :] < lens_a[:, None]
        assert_close(torch.from_numpy(g[mask]), want[mask], what, mag=mag[mask])
    else:
        gs, ws, ms = [], [], []
        for b, h in pairs:
            n = lens_a[b]
            w, m = attn.dense_attention(q[b:b + 1, :, h:h + 1].float().numpy(),
                                        k[b:b + 1, :, h:h + 1].float().numpy(),
                                        v[b:b + 1, :, h:h + 1].float().numpy(), [n], causal, 0.125,
                                        with_magnitude=True)
            gs.append(g[b, :n, h])
            ws.append(w[0, :n, 0])
            ms.append(m[0, :n, 0])
        assert_close(torch.from_numpy(np.concatenate(gs)), np.concatenate(ws), what, mag=np.concatenate(ms))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,T,lens", [(2, 3, 300, [300, 131]), (3, 2, 77, [77, 1, 64]),
                                        (1, 1, 1, [1]), (2, 2, 129, [0, 129]), (1, 2, 128, [128]),
                                        (1, 2, 256, [256]), (2, 1, 257, [257, 250])])
def test_ragged_shapes(gpu, B, H, T, lens, causal):
    import whisper_attention_amd as wa
    announce(f"encoder ragged B={B} H={H} T={T} lens={lens} causal={causal}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=T)
    got = _gpu(wa, q, k, v, lens, causal)
    _check(got, q, k, v, lens, causal, f"encoder B={B} H={H} T={T} causal={causal}")


# Key lengths around the tile edges (64 keys) and around where two key groups
# split a sequence's tiles (the first group takes ceil(tiles / 2)).
EDGE_LENS = [1, 64, 65, 128, 129, 192, 255, 256, 257, 300]


def test_two_key_groups_at_tile_edges(gpu):
    """A grid of few blocks (B*H*query tiles <= 256, 256 keys or more) runs
    two key groups per block, merged in LDS: every key length around a tile
    edge and around the groups' split point, all rows."""
    import whisper_attention_amd as wa
    B, H, T = len(EDGE_LENS), 2, 300
    announce(f"encoder two key groups B={B} H={H} T={T} lens={EDGE_LENS}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=31)
    got = _gpu(wa, q, k, v, EDGE_LENS, False)
    _check(got, q, k, v, EDGE_LENS, False, "encoder two key groups")


def test_one_key_group_at_tile_edges(gpu):
    """The same key lengths on a grid large enough (576 blocks) for one key
    group per block, all rows."""
    import whisper_attention_amd as wa
    B, H, T = 24, 8, 300
    lens = [EDGE_LENS[i % len(EDGE_LENS)] for i in range(B)]
    announce(f"encoder one key group B={B} H={H} T={T}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=32)
    got = _gpu(wa, q, k, v, lens, False)
    _check(got, q, k, v, lens, False, "encoder one key group")


def test_single_chunk_large_v3_all_rows(gpu):
    """One 30-s chunk of the large-v3 shape (B=1, 20 heads, 240 query tiles:
    two key groups per block), every row."""
    import whisper_attention_amd as wa
    announce("encoder B=1 H=20 T=1500")
    q, k, v = workloads.encoder_inputs(1, 20, 1500, seed=33)
    got = _gpu(wa, q, k, v, None, False)
    _check(got, q, k, v, None, False, "encoder B=1 H=20")


def test_long_sequence_two_key_groups(gpu):
    """4096 frames, 2 heads: 64 query tiles, so two key groups per block of
    32 key tiles each (every ring slot many times over); all rows."""
    import whisper_attention_amd as wa
    announce("encoder long sequence B=1 H=2 T=4096")
    q, k, v = workloads.encoder_inputs(1, 2, 4096, seed=35)
    got = _gpu(wa, q, k, v, [4001], False)
    _check(got, q, k, v, [4001], False, "encoder T=4096 two key groups")


def test_long_sequence_causal(gpu):
    """A 3000-token causal prompt, 2 heads: 24 query tiles, each with its own
    diagonal tile and up to 47 key tiles before it; all rows."""
    import whisper_attention_amd as wa
    announce("encoder causal long sequence B=1 H=2 T=3000")
    q, k, v = workloads.encoder_inputs(1, 2, 3000, seed=37)
    got = _gpu(wa, q, k, v, [2950], True)
    _check(got, q, k, v, [2950], True, "encoder causal T=3000")


def test_long_sequence_one_key_group(gpu):
    """4096 frames, 64 heads, B=2 (4096 blocks, one key group): two
    sampled (b, h) checked in full."""
    import whisper_attention_amd as wa
    announce("encoder long sequence B=2 H=64 T=4096")
    q, k, v = workloads.encoder_inputs(2, 64, 4096, seed=36)
    got = _gpu(wa, q, k, v, [4096, 3970], False)
    _check(got, q, k, v, [4096, 3970], False, "encoder T=4096 one key group", pairs=[(0, 0), (1, 63)])


def test_small_workload(gpu):
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["tiny"]
    announce("encoder small workload B=1 H=6 T=1500")
    q, k, v = workloads.encoder_inputs(cfg["B"], cfg["H"], cfg["T"], seed=0)
    got = _gpu(wa, q, k, v, None, False)
    _check(got, q, k, v, None, False, "encoder small")


def test_large_v3_encoder_full_size(gpu):
    """Every (b, h) of the 30-s encoder shape against the oracle, element by
    element: the blocks of one (b, h) are spread over the XCDs by the
    kernel's item order, so a mapping error could touch any of them."""
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["enc_l3"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    announce(f"encoder large-v3 B={B} H={H} T={T} (every (b, h))")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=0)
    got = _gpu(wa, q, k, v, None, False)
    assert torch.isfinite(got.float()).all()
    pairs = [(b, h) for b in range(B) for h in range(H)]
    _check(got, q, k, v, None, False, "encoder large-v3 (every pair)", pairs=pairs)


@pytest.mark.parametrize("name", ["enc_10s", "enc_15s"])
def test_shorter_windows_full_size_sampled(gpu, name):
    """10-s and 15-s chunks (500 and 750 frames) at full batch size."""
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS[name]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    announce(f"encoder {name} B={B} H={H} T={T} (sampled (b, h))")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=0)
    got = _gpu(wa, q, k, v, None, False)
    assert torch.isfinite(got.float()).all()
    g = np.random.default_rng(2)
    pairs = [(0, 0), (B - 1, H - 1)] + [(int(g.integers(B)), int(g.integers(H))) for _ in range(6)]
    _check(got, q, k, v, None, False, f"encoder {name} (sampled)", pairs=pairs)


def test_prefill_causal_full_size(gpu):
    import whisper_attention_amd as wa
    cfg = workloads.CONFIGS["prefill"]
    announce("encoder causal prefill B=128 H=20 T=224 lens U[4,224]")
    q, k, v, lens = workloads.prefill_inputs(cfg["B"], cfg["H"], cfg["T"], cfg["lo"], cfg["hi"],
                                             cfg["outlier_p"], cfg["outlier_mult"], seed=0)
    got = _gpu(wa, q, k, v, lens, True)
    _check(got, q, k, v, lens, True, "prefill causal")


def test_strided_layouts(gpu):
    """Q/K/V stored [B][H][T][64] and passed as [B][T][H][64] views."""
    import whisper_attention_amd as wa
    announce("encoder strided [B][H][T][64] storage")
    B, H, T = 2, 3, 200
    q, k, v = workloads.encoder_inputs(B, H, T, seed=11)
    views = tuple(to_dev(t.permute(0, 2, 1, 3).contiguous()).permute(0, 2, 1, 3) for t in (q, k, v))
    got = _gpu(wa, q, k, v, [200, 150], False, views=views)
    _check(got, q, k, v, [200, 150], False, "encoder strided")


def test_softmax_invariants_on_gpu(gpu):
    """Equal keys -> mean of V; one dominant key -> its V row."""
    import whisper_attention_amd as wa
    announce("encoder softmax invariants")
    T, H = 200, 2
    g = np.random.default_rng(12)
    q = torch.from_numpy(g.standard_normal((1, T, H, 64)).astype(np.float32)).to(torch.bfloat16)
    krow = torch.from_numpy(g.standard_normal(64).astype(np.float32)).to(torch.bfloat16)
    k = krow.expand(1, T, H, 64).contiguous()
    v = torch.from_numpy(g.standard_normal((1, T, H, 64)).astype(np.float32)).to(torch.bfloat16)
    got = _gpu(wa, q, k, v, None, False).float().cpu().numpy()
    mean_v = v.float().numpy().mean(axis=1, keepdims=True)
    assert np.abs(got - mean_v).max() < 2e-2
    k2 = torch.zeros((1, T, H, 64), dtype=torch.bfloat16)
    k2[0, 37, :, 0] = 64.0
    q2 = torch.zeros((1, T, H, 64), dtype=torch.bfloat16)
    q2[..., 0] = 8.0                                 # score 64 * 8 / 8 = 64 vs 0
    got = _gpu(wa, q2, k2, v, None, False).float().cpu().numpy()
    assert np.abs(got - v.float().numpy()[:, 37:38]).max() < 1e-2


@pytest.mark.parametrize("causal", [True, False])
def test_deterministic(gpu, causal):
    """Two calls give the same bits: causal (one key group) and non-causal at
    this size (B*H*query tiles = 48, two key groups merged in LDS)."""
    import whisper_attention_amd as wa
    announce(f"encoder determinism causal={causal}")
    q, k, v = workloads.encoder_inputs(2, 4, 700, seed=13)
    a = _gpu(wa, q, k, v, [700, 333], causal)
    b = _gpu(wa, q, k, v, [700, 333], causal)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lam", [4.0, 10.0, 20.0, 100.0])
def test_late_large_scores(gpu, lam, causal):
    """Keys of later tiles scaled by lam: the scores of those tiles exceed
    the earlier tiles' by about 4*lam bits (exp2 domain), so the running max
    jumps in the middle of a row (and, for lam = 4, may stay within the
    kernel's headroom above its reference, so no redo) -- in a full middle
    tile, in one key of an early tile and in the ragged last tile."""
    import whisper_attention_amd as wa
    B, H, T = 2, 2, 700
    announce(f"encoder late large scores lam={lam} causal={causal}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=11)
    kf = k.float()
    kf[0, 400:464] *= lam          # a whole middle tile
    kf[0, 130:131] *= lam          # one key of an early tile
    kf[1, 640:700] *= lam          # the ragged last tile
    k = kf.to(torch.bfloat16)
    lens = [700, 690]
    got = _gpu(wa, q, k, v, lens, causal)
    _check(got, q, k, v, lens, causal, f"late large scores lam={lam} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores_redo_every_tile(gpu, causal):
    """The keys of tile j scaled by 1 + 2.5 j: each tile's largest score
    exceeds the previous tile's by more than the kernel's headroom above its
    reference (8 log2 units), so nearly every tile's weights reach 2 against
    the reference and the tile is redone with its exact max, rescaling O and
    the row sums each time; the early tiles' weights end up below fp32's
    range, as they are below the oracle's rounding.  Ragged last tile."""
    import whisper_attention_amd as wa
    B, H, T = 2, 3, 1500
    announce(f"encoder rising scores, every tile redone, causal={causal}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=12)
    kf = k.float()
    for j in range((T + 63) // 64):
        kf[:, j * 64:(j + 1) * 64] *= 1.0 + 2.5 * j
    k = kf.to(torch.bfloat16)
    lens = [1500, 1471]
    got = _gpu(wa, q, k, v, lens, causal)
    _check(got, q, k, v, lens, causal, f"rising scores causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_every_ring_position(gpu, causal):
    """Key ranges of 1 to 14 tiles, whole and ragged, in one batch: the loop
    over key tiles (two K slots, three V slots, unrolled by six) ends at
    every position of its unrolled body, and the query tiles (128 rows)
    end at every wave."""
    import whisper_attention_amd as wa
    lens = [64 * n + r for n in range(14) for r in (0, 17) if 64 * n + r > 0]
    B, H, T = len(lens), 2, max(lens)
    announce(f"every ring position, causal={causal}: B={B} T={T} lens={lens}")
    q, k, v = workloads.encoder_inputs(B, H, T, seed=31)
    got = _gpu(wa, q, k, v, lens, causal)
    _check(got, q, k, v, lens, causal, f"ring positions causal={causal}")
