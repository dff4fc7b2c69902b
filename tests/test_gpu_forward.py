"""GPU parity of the forward path (encode, merge, decode, FLARE, FLARE++) against the CPU oracle.

Every case draws seeded inputs (workloads), runs the HIP library through its
C ABI, copies the very same input bits to the host for the float64 oracle and
compares element by element.  Sizes span several 64-token tiles, ragged
partition tails and empty partitions.
"""
import numpy as np
import pytest
import torch

import split_kv_softmax_amd as fl
import workloads as W
from oracle import flare_ref as ref
from tests._util import F32_ATOL, compare, compare_bf16, compare_L, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _enc_case(M, D, N, R, B=2, H=2, dtype="bf16", masked=False, q_per_batch=False, stress=1.0, wid=500):
    base = W.Workload(name=f"case_M{M}_D{D}_N{N}", wid=wid + M + D, kind="encode", dtype=dtype, B=B, H=H, N=N,
                      M=M, D=D, offsets=W.ragged_offsets(N, R, wid + M + D), q_std=D ** -0.5,
                      q_per_batch=q_per_batch, stress=stress)
    # make sure at least one partition is empty
    offs = list(base.offsets)
    if R >= 3:
        offs[2] = offs[1]
    base = base.with_(offsets=offs)
    x = base.make(DEV)
    if masked:
        g = np.random.default_rng(wid)
        m = (g.random((B, N)) > 0.35).astype(np.uint8)
        m[:, 0] = 1
        # one partition fully masked for batch 0
        if R >= 4:
            m[0, offs[3]:offs[4]] = 0
        x["mask"] = torch.from_numpy(m).to(DEV)
    return base, x


def _check_encode(w, x, fp32=False, report=None):
    mask = x.get("mask")
    O_part, L_part = fl.encode(x["Q"], x["K"], x["V"], w.offsets, mask, w.scale)
    Z, L, _ = fl.lse_merge(O_part, L_part)
    torch.cuda.synchronize()
    out = ref.encode_ref(x["Q"], x["K"], x["V"], w.offsets, mask, w.scale)
    if fp32:
        compare(O_part, out["O_part"], "O_part", F32_ATOL, report=report)
        compare(L_part, out["L_part"], "L_part", F32_ATOL, report=report)
        compare(Z, out["Z"], "Z", F32_ATOL, report=report)
        compare(L, out["L"], "L", F32_ATOL, report=report)
    else:
        compare_bf16(O_part, out["O_part"], "O_part", report)
        compare_L(L_part, out["L_part"], "L_part", report=report)
        compare_bf16(Z, out["Z"], "Z", report)
        compare_L(L, out["L"], "L", report=report)
    return O_part, L_part, Z, L, out


def test_fp32_small_encoder_workload():
    """The single-head fp32 encoder with partitions 300/200/424/100 (max-abs 1e-5)."""
    w = W.FLARE_ENCODE_F32_SMALL
    x = w.make(DEV)
    _check_encode(w, x, fp32=True)


@pytest.mark.parametrize("M,D", [(32, 64), (64, 64), (128, 64), (256, 64), (32, 128), (64, 128), (128, 128),
                                 (256, 128), (32, 16), (64, 16), (128, 16), (256, 16)])
@pytest.mark.parametrize("masked", [False, True])
def test_bf16_encoder_matrix_core(M, D, masked):
    # head dim 16 at 64 or 128 latent rows without a mask takes the pipelined encoder
    w, x = _enc_case(M, D, N=2500, R=5, masked=masked)
    _check_encode(w, x)


@pytest.mark.parametrize("M,D", [(128, 16), (64, 16), (128, 64)])
def test_far_negative_and_large_scores(M, D):
    """Rows whose every score sits near -300 (so a weight against a zero reference underflows and
    the row must re-base downwards), rows with score spread ~30 (re-base upwards), and ordinary
    rows, through the unmasked pipelined encoder (head dim 16 folds the scale and the reference
    into the score products): parity with the oracle, L within the bf16 bound."""
    w, x = _enc_case(M, D, N=3000, R=4, wid=720)
    Q = x["Q"].float().clone()
    K = x["K"].float().clone()
    c = 12.0 if D == 16 else 16.0
    K[..., 0] = c                                   # every key has a large first coordinate
    Q[:, : M // 4, :] = 0.0
    Q[:, : M // 4, 0] = -c                          # rows 0..M/4-1: every score = -s c^2 (about -36..-32 s^-1)
    Q[:, M // 4: M // 2] *= 8.0 * D ** 0.5          # rows M/4..M/2-1: wide spread
    x["Q"] = Q.to(torch.bfloat16)
    x["K"] = K.to(torch.bfloat16)
    # the scale puts the first quarter's scores at about -300 (natural units)
    sc = float(np.float32(300.0 / (c * c)))
    O_part, L_part = fl.encode(x["Q"], x["K"], x["V"], w.offsets, None, sc)
    Z, L, _ = fl.lse_merge(O_part, L_part)
    torch.cuda.synchronize()
    out = ref.encode_ref(x["Q"], x["K"], x["V"], w.offsets, None, sc)
    compare_bf16(O_part, out["O_part"], "O_part")
    compare_L(L_part, out["L_part"], "L_part")
    compare_bf16(Z, out["Z"], "Z")
    compare_L(L, out["L"], "L")
    assert float(L[0, 0, 0]) < -250.0


def test_bf16_encoder_stress_scores():
    """Q scaled so score spread is ~4: exercises the running-max rescale."""
    w, x = _enc_case(128, 64, N=3000, R=4, stress=4 * 8.0)
    _check_encode(w, x)


def test_bf16_encoder_split_partitions():
    """Long partitions split into several chunks and folded by the library."""
    w = W.shrink(W.FLAREPP, 40000, R=2, H=2)
    x = {"Q": W.normal((2, 128, 64), 77, W.T_Q, 1 / 8, torch.bfloat16, DEV),
         "K": W.normal((1, 2, 40000, 64), 77, W.T_K, 1.0, torch.bfloat16, DEV),
         "V": W.normal((1, 2, 40000, 64), 77, W.T_V, 1.0, torch.bfloat16, DEV)}
    w = w.with_(kind="encode")
    nbytes = fl.encode_workspace_size(torch.bfloat16, 1, 2, 40000, 128, 64, w.offsets)
    assert nbytes > 0, "expected the library to split these partitions"
    _check_encode(w, x)


@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("D", [64, 16])
def test_bf16_encoder_partitions_shorter_than_a_tile_per_group(masked, D):
    """Partitions of 1, 63, 64, 65, 127, 128, 129 and 0 tokens: fewer 64-token
    tiles than the encoder's token groups, partial last tiles, an empty one."""
    offs = [0, 1, 64, 128, 193, 320, 448, 577, 577, 800]
    w, x = _enc_case(128, D, N=offs[-1], R=len(offs) - 1, masked=masked)
    w = w.with_(offsets=offs)
    if masked:
        x["mask"][:, 1:64] = 1          # keep the 63-token partition fully valid
    _check_encode(w, x)


def test_nan_query_row_stays_in_its_row():
    """A NaN in one latent query row makes only that row NaN (the oracle says so);
    rows whose weights share a matrix-core product with it stay exact."""
    for M, masked in ((128, False), (128, True), (64, False)):
        w, x = _enc_case(M, 64, N=1300, R=3, masked=masked)
        x["Q"][:, 5] = float("nan")
        _check_encode(w, x)             # NaN reference entries are skipped, every other one compared
        O_part, _ = fl.encode(x["Q"], x["K"], x["V"], w.offsets, x.get("mask"), w.scale)
        torch.cuda.synchronize()
        o = O_part.cpu()
        assert not torch.isnan(o[:, :, :, 21]).any() and not torch.isnan(o[:, :, :, 37]).any()


def test_decode_nan_token_stays_in_its_row():
    """An unmasked token row holding NaN gives NaN only in its own output row."""
    B, H, N, M, D = 1, 2, 300, 128, 64
    Xq = W.normal((B, H, N, D), 612, W.T_K, 1.0, torch.bfloat16, DEV)
    Xq[0, :, 40] = float("nan")
    Kl = W.normal((H, M, D), 612, W.T_Q, 1.0, torch.bfloat16, DEV)
    Z = W.normal((B, H, M, D), 612, W.T_V, 1.0, torch.float32, DEV)
    Y = fl.decode(Xq, Kl, Z, 0.125)
    torch.cuda.synchronize()
    Yc = Y.float().cpu()
    assert torch.isnan(Yc[0, :, 40]).all()
    ref_y = ref.decode_ref(Xq, Kl, Z, 0.125)           # NaN in row 40 only
    compare_bf16(Y, ref_y, "Y")


@pytest.mark.parametrize("D", [32, 64, 128])
def test_single_query_split_kv(D):
    w, x = _enc_case(1, D, N=5000, R=7, B=2, H=3, q_per_batch=True)
    _check_encode(w, x)


def test_generic_vector_path_bf16():
    """A bf16 shape without a matrix-core variant (M=16) takes the vector path."""
    w, x = _enc_case(16, 64, N=700, R=3, masked=True)
    _check_encode(w, x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,D", [(5, 128), (5, 256), (7, 64), (3, 32)])
@pytest.mark.parametrize("masked", [False, True])
def test_vector_path_wide_heads_and_partial_row_groups(M, D, dtype, masked):
    """The vector encoder at head dims above 64 (32- and 16-token tiles, several lanes per
    head dim) and M not a multiple of 4 (inactive waves), ragged partitions with an empty
    one, masked and not; float32 to max-abs 1e-5, bfloat16 to the bf16 bounds."""
    w, x = _enc_case(M, D, N=1100, R=4, dtype=dtype, masked=masked, wid=700)
    _check_encode(w, x, fp32=dtype == "f32")


def test_nan_padding_never_leaks_vector_path():
    """NaN keys and Inf values in padded slots, float32 through the vector encoder: the states
    are bitwise those of clean padding (padded rows are zero rows in the staged tile)."""
    w, x = _enc_case(16, 32, N=1500, R=4, dtype="f32", masked=True, wid=710)
    inv = (x["mask"] == 0)[:, None, :, None].expand_as(x["K"])
    K2 = x["K"].masked_fill(inv, float("nan"))
    V2 = x["V"].masked_fill(inv, float("inf"))
    a = fl.encode(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale)
    b = fl.encode(x["Q"], K2, V2, w.offsets, x["mask"], w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.isnan(b[0]).any()
    _check_encode(w, x, fp32=True)


def test_fp32_generic_larger():
    w, x = _enc_case(24, 32, N=1500, R=4, dtype="f32", masked=True)
    _check_encode(w, x, fp32=True)


# ------------------------------------------------------------------- decode
@pytest.mark.parametrize("M,D", [(32, 64), (64, 64), (128, 64), (256, 64), (32, 128), (64, 128), (128, 128),
                                 (256, 128), (32, 16), (64, 16), (128, 16), (256, 16)])
def test_decode_matrix_core(M, D):
    B, H, N = 2, 2, 1000
    Xq = W.normal((B, H, N, D), 600 + M, W.T_K, 1.0, torch.bfloat16, DEV)
    Kl = W.normal((H, M, D), 600 + M, W.T_Q, 1.0, torch.bfloat16, DEV)
    Z = W.normal((B, H, M, D), 600 + M, W.T_V, 1.0, torch.float32, DEV)
    s = W.scale_for(D)
    Y = fl.decode(Xq, Kl, Z, s)
    torch.cuda.synchronize()
    compare_bf16(Y, ref.decode_ref(Xq, Kl, Z, s), "Y")


def test_decode_token_mask_and_fp32():
    B, H, N, M, D = 2, 3, 333, 20, 32
    Xq = W.normal((B, H, N, D), 610, W.T_K, 1.0, torch.float32, DEV)
    Kl = W.normal((B, H, M, D), 610, W.T_Q, 1.0, torch.float32, DEV)
    Z = W.normal((B, H, M, D), 610, W.T_V, 1.0, torch.float32, DEV)
    tm = (torch.rand(B, N, generator=torch.Generator().manual_seed(3)) > 0.3).to(torch.uint8).to(DEV)
    Y = fl.decode(Xq, Kl, Z, 0.2, token_mask=tm)
    torch.cuda.synchronize()
    compare(Y, ref.decode_ref(Xq, Kl, Z, 0.2, token_mask=tm), "Y", F32_ATOL)


def test_decode_token_mask_bf16():
    B, H, N, M, D = 1, 2, 500, 128, 64
    Xq = W.normal((B, H, N, D), 611, W.T_K, 1.0, torch.bfloat16, DEV)
    Xq[0, :, 7] = float("nan")          # a padded token's row may hold anything
    Kl = W.normal((H, M, D), 611, W.T_Q, 1.0, torch.bfloat16, DEV)
    Z = W.normal((B, H, M, D), 611, W.T_V, 1.0, torch.float32, DEV)
    tm = torch.ones(B, N, dtype=torch.uint8, device=DEV)
    tm[0, 7] = 0
    tm[0, 100:140] = 0
    Y = fl.decode(Xq, Kl, Z, 0.125, token_mask=tm)
    torch.cuda.synchronize()
    compare_bf16(Y, ref.decode_ref(Xq.nan_to_num(0.0), Kl, Z, 0.125, token_mask=tm), "Y")


# ------------------------------------------------------------ FLARE / FLARE++
def test_flare_block_small():
    w = W.shrink(W.FLARE_BLOCK, 6000, R=8, B=2, H=2, ragged=True)
    x = w.make(DEV)
    out = fl.flare_forward(x["Q"], x["K"], x["V"], w.offsets, None, w.scale)
    torch.cuda.synchronize()
    e = ref.encode_ref(x["Q"], x["K"], x["V"], w.offsets, None, w.scale)
    compare_bf16(out["Z"], e["Z"], "Z")
    compare_L(out["L"], e["L"], "L")
    compare_bf16(out["Y"], ref.decode_ref(x["K"], x["Q"], e["Z"], w.scale), "Y")


def test_flarepp_small():
    w = W.shrink(W.FLAREPP, 5000, R=4, H=2, ragged=True)
    x = w.make(DEV)
    out = fl.flarepp_forward(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale)
    torch.cuda.synchronize()
    r = ref.flarepp_ref(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale)
    compare_bf16(out["QX"], r["QX"], "QX")
    compare_bf16(out["Z"], r["Z"], "Z")
    compare_L(out["L"], r["L"], "L")
    compare_bf16(out["Y"], r["Y"], "Y")


def test_flarepp_head_dim_16_small():
    """The FLARE++ chain at head dim 16 (the pages' C = 128, H = 8 backbone), ragged partitions."""
    w = W.shrink(W.FLAREPP_D16, 6000, R=5, H=3, ragged=True)
    x = w.make(DEV)
    out = fl.flarepp_forward(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale)
    torch.cuda.synchronize()
    r = ref.flarepp_ref(x["Qt"], x["Kt"], x["Vt"], x["K"], x["V"], w.offsets, w.scale)
    compare_bf16(out["QX"], r["QX"], "QX")
    compare_bf16(out["Z"], r["Z"], "Z")
    compare_L(out["L"], r["L"], "L")
    compare_bf16(out["Y"], r["Y"], "Y")


def test_encoder_head_dim_16_split_partitions_and_one_call():
    """Head dim 16 with partitions cut into chunks (few slices), and the one-call form bit for bit."""
    w = W.shrink(W.FLAREPP_D16, 40000, R=2, H=1, ragged=True)
    x = w.make(DEV)
    O, Lp, Z, L, Zb = fl.encode_merge(x["Qt"], x["K"], x["V"], w.offsets, None, w.scale, True)
    O2, Lp2 = fl.encode(x["Qt"], x["K"], x["V"], w.offsets, None, w.scale)
    Z2, L2, Zb2 = fl.lse_merge(O2, Lp2, want_bf16=True)
    torch.cuda.synchronize()
    for a, b, n in ((O, O2, "O_part"), (Lp, Lp2, "L_part"), (Z, Z2, "Z"), (L, L2, "L"), (Zb, Zb2, "Z_bf16")):
        assert torch.equal(a, b), n
    e = ref.encode_ref(x["Qt"], x["K"], x["V"], w.offsets, None, w.scale)
    compare_bf16(O, e["O_part"], "O_part")
    compare_L(Lp, e["L_part"], "L_part")
    compare_bf16(Z, e["Z"], "Z")
    compare_L(L, e["L"], "L")


# ------------------------------------------------------- exactness properties
def test_empty_and_fully_masked_partitions_are_exact():
    w, x = _enc_case(64, 64, N=1200, R=5, masked=True)
    O_part, L_part = fl.encode(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale)
    torch.cuda.synchronize()
    o = O_part.cpu()
    l = L_part.cpu()
    assert torch.isneginf(l[1]).all()                          # empty by offsets
    assert (o[1] == 0).all() and not torch.signbit(o[1]).any()
    assert torch.isneginf(l[3, 0]).all() and (o[3, 0] == 0).all()   # fully masked, batch 0
    assert not torch.isnan(o).any()


def test_nan_padding_never_leaks():
    w, x = _enc_case(128, 64, N=1500, R=4, masked=True)
    inv = (x["mask"] == 0)[:, None, :, None].expand_as(x["K"])
    K2 = x["K"].masked_fill(inv, float("nan"))
    V2 = x["V"].masked_fill(inv, float("inf"))
    a = fl.encode(x["Q"], x["K"], x["V"], w.offsets, x["mask"], w.scale)
    b = fl.encode(x["Q"], K2, V2, w.offsets, x["mask"], w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.isnan(b[0]).any()


def test_runs_are_bitwise_deterministic():
    w, x = _enc_case(128, 64, N=9000, R=3)
    a = fl.flare_forward(x["Q"], x["K"], x["V"], w.offsets)
    b = fl.flare_forward(x["Q"], x["K"], x["V"], w.offsets)
    torch.cuda.synchronize()
    for k in ("O_part", "L_part", "Z", "L", "Y"):
        assert torch.equal(a[k], b[k]), k


# ------------------------------------------------------------ spike tests
def _spike_inputs(B, H, N, M, D, spikes, device=DEV, dtype=torch.bfloat16):
    """Q[m] = a e_{m mod D}; K[n*] = a e_j for each (n*, j) spike, 0 elsewhere;
    V rows carry (n mod 256, n // 256 mod 256, h, b) as bf16-exact integers."""
    a = 32.0 if D <= 64 else 64.0
    Q = torch.zeros(H, M, D)
    for m in range(M):
        Q[:, m, m % D] = a
    K = torch.zeros(B, H, N, D)
    for n, j in spikes:
        K[:, :, n, j] = a
    n_idx = torch.arange(N, dtype=torch.float32)
    V = torch.zeros(B, H, N, D)
    V[..., 0] = (n_idx % 256)[None, None]
    V[..., 1] = ((n_idx // 256) % 256)[None, None]
    V[..., 2] = torch.arange(H, dtype=torch.float32)[None, :, None]
    V[..., 3] = torch.arange(B, dtype=torch.float32)[:, None, None]
    return (Q.to(dtype).to(device), K.to(dtype).to(device), V.to(dtype).to(device))


@pytest.mark.parametrize("M,D", [(64, 64), (128, 64), (256, 128), (1, 128), (64, 16), (128, 16)])
def test_spike_index_handling_is_bit_exact(M, D):
    B, H = 2, 3
    offs = [0, 300, 500, 500, 924, 1024, 1500]
    N = offs[-1]
    # spikes at partition edges and tile tails, one direction each
    positions = [0, 299, 300, 499, 500, 563, 923, 924, 1023, 1024, 1087, 1499]
    dirs = list(range(len(positions)))
    spikes = list(zip(positions, dirs))
    Q, K, V = _spike_inputs(B, H, N, M, D, spikes)
    if M == 1:
        Q = Q[:, :1].unsqueeze(0).expand(B, H, 1, D).contiguous()
        Q[:] = 0
        Q[..., 5] = 32.0 if D <= 64 else 64.0         # row 0 looks for direction 5 -> token 923
    s = W.scale_for(D)
    O_part, L_part = fl.encode(Q, K, V, offs, None, s)
    Z, L, _ = fl.lse_merge(O_part, L_part)
    torch.cuda.synchronize()
    Zc, Vc = Z.cpu(), V.float().cpu()
    for m in range(M):
        j = (m % D) if M > 1 else 5
        if j >= len(positions):
            continue
        n_star = positions[j]
        r_star = max(r for r in range(len(offs) - 1) if offs[r] <= n_star < offs[r + 1])
        assert torch.equal(Zc[:, :, m], Vc[:, :, n_star]), (m, n_star)
        assert torch.equal(O_part[r_star, :, :, m].cpu(), Vc[:, :, n_star]), (m, n_star, r_star)
    # empty partition 2 is exactly (0, -inf)
    assert torch.isneginf(L_part[2]).all() and (O_part[2] == 0).all()
    if M > 1:
        # decode: spike token n*_j attends only to latents with direction j
        Y = fl.decode(K, Q, Z, s)
        torch.cuda.synchronize()
        Yc = Y.float().cpu()
        for j, n_star in enumerate(positions):
            if j >= min(M, D):
                continue
            assert torch.equal(Yc[:, :, n_star], Zc[:, :, j]), (j, n_star)


@pytest.mark.parametrize("M", [16, 5])
def test_spike_index_handling_fp32_vector_path(M):
    """The float32 small-encoder shape (partitions 300/200/424/100, vector kernel with its
    64-token tiles and 128-token chunks): spikes at partition edges and tile tails give
    O_r[m] = V[n*] and Z[m] = V[n*] bit for bit, L_r = s a^2 to 2 ulp, and the spike of a
    masked slot is ignored.  M = 5 leaves inactive waves in the last group of four rows."""
    B, H, N, D = 1, 1, 1024, 32
    offs = [0, 300, 500, 924, 1024]
    positions = [0, 63, 64, 127, 128, 299, 300, 499, 500, 923, 924, 1023]
    spikes = list(zip(positions, range(len(positions))))
    Q, K, V = _spike_inputs(B, H, N, M, D, spikes + [(700, 0)], dtype=torch.float32)
    Q = Q.unsqueeze(0).contiguous()          # the small encoder's Q is per batch
    mask = torch.ones(B, N, dtype=torch.uint8, device=DEV)
    mask[:, 700] = 0                          # a padded decoy in direction 0
    s = float(np.float32(D ** -0.5))
    O_part, L_part = fl.encode(Q, K, V, offs, mask, s)
    Z, L, _ = fl.lse_merge(O_part, L_part)
    torch.cuda.synchronize()
    Vc = V.cpu()
    want_L = float(np.float32(s) * np.float32(32.0 * 32.0))
    for m in range(min(M, len(positions))):
        n_star = positions[m]
        r_star = max(r for r in range(len(offs) - 1) if offs[r] <= n_star < offs[r + 1])
        assert torch.equal(O_part[r_star, :, :, m].cpu(), Vc[:, :, n_star]), (m, n_star)
        assert torch.equal(Z[:, :, m].cpu(), Vc[:, :, n_star]), (m, n_star)
        assert abs(float(L_part[r_star, 0, 0, m]) - want_L) <= 2 * np.spacing(np.float32(want_L)), m
        for r in range(len(offs) - 1):
            if r != r_star:
                # no spike of its direction here: every score is 0, O is the partition's mean of V
                assert float(L_part[r, 0, 0, m]) < 10.0


def test_uniform_scores_give_mean_of_v_on_gpu():
    """Q = 0: every valid score is 0, so Z is the mean of the valid V rows and L = ln(count)."""
    w, x = _enc_case(64, 64, N=1000, R=4, masked=True)
    Q = torch.zeros_like(x["Q"])
    O_part, L_part = fl.encode(Q, x["K"], x["V"], w.offsets, x["mask"], w.scale)
    Z, L, _ = fl.lse_merge(O_part, L_part)
    torch.cuda.synchronize()
    m = x["mask"].cpu().bool()
    V = to64(x["V"])
    for b in range(w.B):
        cnt = int(m[b].sum())
        np.testing.assert_allclose(to64(L[b]), np.log(cnt), rtol=0, atol=1e-5)
        mean = V[b][:, m[b].numpy()].mean(axis=1)       # [H, D]
        np.testing.assert_allclose(to64(Z[b]), np.broadcast_to(mean[:, None, :], Z[b].shape), rtol=0, atol=1e-5)
