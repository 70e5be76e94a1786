"""GPU parity at the full layer sizes of every workload, on sampled outputs (marker `gpu`).

The GPU runs the whole path exactly as the benchmark launches it (set-up, merge,
activation quantization, integer linear layer over all rows and tokens).  Every step
of set-up and merge is row-local (per-row statistics; R depends on (seed, layer, i, j)
only), so the oracle recomputes a sample of rows from the raw inputs of those rows
alone, and the linear layer's outputs at (sampled token, sampled row) pairs.  All
sampled values must be bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
from integer_rank_adaptation_amd import synth
from tests.test_gpu_parity import bits, cuda, host, unpack4, unpack4s

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from integer_rank_adaptation_amd import ops as _ops

    _ops.B.lib()
    return _ops


def sample_rows(d, k, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = {0, d - 1} | set(rng.choice(d, size=min(k, d), replace=False).tolist())
    return np.array(sorted(rows))


def check_layer(ops, wl, li, L, Ms, mode, mbits, block=0, n_rows=6, n_tok=6):
    lid = synth.layer_id(wl.index, li, block)
    W = synth.weight(wl, li, block=block)
    A, Bm = synth.lora(wl, li, block=block)
    seed = synth.PHILOX_SEED
    st = ops.setup_layer(cuda(W), wl.w_bits, seed, lid, synth.ALPHA)
    if mode == "mul":
        g = ops.merge_mul(st, cuda(A), cuda(Bm), wl.w_bits, mbits, seed, lid, dbg=True)
    else:
        g = ops.merge_shift(st, cuda(A), cuda(Bm), wl.w_bits, mbits, seed, lid, dbg=True)
    rows = sample_rows(L.d, n_rows, 7 * li + block)
    # oracle on the sampled rows only (row-local set-up and merge)
    sig = oracle.sigma_w(W[rows])
    c = oracle.vmc_scale(sig, synth.ALPHA)
    R = np.concatenate([oracle.gen_r_rows(int(i), 1, L.n, seed, lid, c[k:k + 1]) for k, i in enumerate(rows)])
    wr, z, s = oracle.base_quant(W[rows], R, wl.w_bits)
    gwr = host(st["wround"])
    gwr = unpack4(gwr) if wl.w_bits == 4 else gwr
    assert np.array_equal(bits(host(st["c"])[rows]), bits(c))
    assert np.array_equal(gwr[rows], wr)
    assert np.array_equal(host(st["z"])[rows], z)
    assert np.array_equal(bits(host(st["s"])[rows]), bits(s))
    gp = None
    if mode == "mul":
        ref = oracle.merge_mul(wr, z, s, R, A[rows], Bm, mbits)
        if L.n % 16 == 0:  # the byte-plane storage the benchmark's step uses
            gp = ops.merge_mul_planes(st, cuda(A), cuda(Bm), wl.w_bits, mbits, seed, lid)
            lay, code = oracle.plane_store(ref["m"], z, ref["zbar"], wl.w_bits, mbits)
            assert np.array_equal(host(gp["code"])[rows], code)
            assert np.array_equal(host(gp["planes"])[rows], lay)
        m_all = host(g["m"])
        assert np.array_equal(host(g["uround"])[rows], ref["uround"])
        assert np.array_equal(host(g["zbar"])[rows], ref["zbar"])
        assert np.array_equal(host(g["split"])[rows], oracle.plane_split(ref["m"]))
        m_rows = m_all[rows]
        wfmt = 16
    else:
        ref = oracle.merge_shift(wr, z, s, R, A[rows], Bm, wl.w_bits, mbits)
        m_all = host(g["m"])
        m_all = unpack4s(m_all) if wl.w_bits == 4 else m_all.view(np.int8)
        m_rows = m_all[rows]
        assert np.array_equal(host(g["shift"])[rows], ref["shift"])
        wfmt = wl.w_bits
    assert np.array_equal(m_rows, ref["m"]), (wl.name, L.name, mode)
    assert np.array_equal(bits(host(g["sbar"])[rows]), bits(ref["sbar"]))
    # linear layer: every token and output on the GPU; oracle at sampled (t, i)
    for M in Ms:
        X = synth.activations(wl, L.n, M, li)
        xq, sx, rs = ops.quant_act(cuda(X))
        Y, _ = ops.linear(xq, sx, rs, wfmt, g["m"], g["sbar"], L.d, split=g.get("split"))
        if mode == "mul":  # the bias split on every row gives the same outputs
            Yb, _ = ops.linear(xq, sx, rs, wfmt, g["m"], g["sbar"], L.d)
            assert torch.equal(Y, Yb), (wl.name, L.name, M)
        if gp is not None:  # and so do the byte planes
            Yp, _ = ops.linear(xq, sx, rs, ops.B.INTLORA_W_INT16_PLANES, gp["planes"], gp["sbar"], L.d,
                               split=gp["code"])
            assert torch.equal(Y, Yp), (wl.name, L.name, M)
        toks = sample_rows(M, n_tok, 11 * li + M)
        oxq, osx, _ = oracle.quant_act(X[toks])
        assert np.array_equal(host(xq)[toks], oxq)
        assert np.array_equal(bits(host(sx)[toks]), bits(osx))
        tt, ii = np.meshgrid(np.arange(toks.size), np.arange(rows.size), indexing="ij")
        exact, y = oracle.linear_sampled(tt.ravel(), ii.ravel(), oxq, osx, ref["m"].astype(np.int32), ref["sbar"])
        Yh = host(Y).view(np.uint16)
        got = Yh[np.ix_(toks, rows)].ravel()
        assert np.array_equal(got, y), (wl.name, L.name, mode, M)
    return int(host(g["sat"])[0])


@pytest.mark.parametrize("wl_index", [0, 1, 2, 3, 4])
def test_workload_full_size_sampled(ops, wl_index):
    wl = synth.WORKLOADS[wl_index]
    for li, L in enumerate(wl.layers):
        for mode, mbits in wl.modes:
            check_layer(ops, wl, li, L, wl.tokens, mode, mbits)
        torch.cuda.empty_cache()


@pytest.mark.parametrize("block", [1, 31])
def test_llama_sweep_blocks_sampled(ops, block):
    """The merge-only sweep of the Llama-shaped workload: other transformer blocks use
    other layer ids (7 * block + matrix); sampled rows of every matrix."""
    wl = synth.WORKLOADS[4]
    mode, mbits = wl.modes[0]
    for li, L in enumerate(wl.layers):
        check_layer(ops, wl, li, L, (16,), mode, mbits, block=block, n_rows=4, n_tok=2)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wl_index,li", [(3, 0), (3, 3), (4, 4)])
def test_ptq_path_full_size_sampled(ops, wl_index, li):
    """The QLoRA-style comparison path at full layer size (FLUX qkv and mlp_out, Llama
    gate): sampled rows of codes, s' and z' equal the oracle's, at the base's bit width."""
    wl = synth.WORKLOADS[wl_index]
    L = wl.layers[li]
    lid = synth.layer_id(wl.index, li)
    W = synth.weight(wl, li)
    A, Bm = synth.lora(wl, li)
    seed = synth.PHILOX_SEED
    st = ops.setup_layer(cuda(W), wl.w_bits, seed, lid, synth.ALPHA)
    g = ops.merge_ptq(st, cuda(A), cuda(Bm), wl.w_bits, wl.w_bits, seed, lid)
    rows = sample_rows(L.d, 6, 13 * li + wl_index)
    sig = oracle.sigma_w(W[rows])
    c = oracle.vmc_scale(sig, synth.ALPHA)
    R = np.concatenate([oracle.gen_r_rows(int(i), 1, L.n, seed, lid, c[k:k + 1]) for k, i in enumerate(rows)])
    wr, z, s = oracle.base_quant(W[rows], R, wl.w_bits)
    ref = oracle.ptq_merge(wr, z, s, R, A[rows], Bm, wl.w_bits)
    code = host(g["code"])
    code = unpack4(code) if wl.w_bits == 4 else code
    assert np.array_equal(code[rows], ref["code"])
    assert np.array_equal(bits(host(g["s"])[rows]), bits(ref["s"]))
    assert np.array_equal(host(g["z"])[rows], ref["z"])
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wl_index,li", [(3, 0), (3, 3), (4, 6)])
def test_ste_backward_full_size(ops, wl_index, li):
    """The straight-through backward at full layer size (FLUX qkv and mlp_out, Llama
    down): every output of dA and dB within the binary32 summation bound of the binary64
    oracle."""
    from oracle import algebra

    wl = synth.WORKLOADS[wl_index]
    L = wl.layers[li]
    lid = synth.layer_id(wl.index, li)
    W = synth.weight(wl, li)
    A, Bm = synth.lora(wl, li)
    G = synth.random_matrix(900 + li, (L.d, L.n), 1e-3)
    st = ops.setup_layer(cuda(W), wl.w_bits, synth.PHILOX_SEED, lid, synth.ALPHA)
    g = ops.ste_backward(st, cuda(A), cuda(Bm), cuda(G), wl.w_bits)
    wr = host(st["wround"])
    wr = unpack4(wr) if wl.w_bits == 4 else wr
    z = host(st["z"])
    rA, rB = algebra.ste_backward(wr, z, A, Bm, G)
    absD = np.abs(G.astype(np.float64)) * ((wr.astype(np.int64) - z.astype(np.int64)[:, None]) != 0)
    boundA = (L.n + 16) * 2.0**-23 * (absD @ np.abs(Bm.astype(np.float64)).T) + 1e-30
    boundB = (L.d + 16) * 2.0**-23 * (np.abs(A.astype(np.float64)).T @ absD) + 1e-30
    assert np.all(np.abs(host(g["dA"]).astype(np.float64) - rA) <= boundA)
    assert np.all(np.abs(host(g["dB"]).astype(np.float64) - rB) <= boundB)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("li", [0, 3])
def test_merge_on_load_full_size(ops, li):
    """FLUX qkv (9216 x 3072) and mlp_out (3072 x 12288) at full size, 4608 tokens: the
    merge keeping U's codes stores exactly the MUL merge's U_round, and the merge-on-load
    linear layer gives the INT16 path's outputs bit for bit; sampled outputs against the
    oracle on m formed from the codes."""
    wl = synth.WORKLOADS[3]
    L = wl.layers[li]
    M = wl.tokens[0]
    lid = synth.layer_id(wl.index, li)
    seed = synth.PHILOX_SEED
    W = synth.weight(wl, li)
    A, Bm = synth.lora(wl, li)
    st = ops.setup_layer(cuda(W), wl.w_bits, seed, lid, synth.ALPHA)
    _, ubits = wl.modes[0]
    g = ops.merge_mul(st, cuda(A), cuda(Bm), wl.w_bits, ubits, seed, lid, dbg=True)
    gc = ops.merge_mul_codes(st, cuda(A), cuda(Bm), wl.w_bits, ubits, seed, lid)
    ucode = unpack4(host(gc["ucode"]))
    assert np.array_equal(ucode, host(g["uround"]))
    assert np.array_equal(host(gc["zbar"]), host(g["zbar"]))
    assert np.array_equal(bits(host(gc["sbar"])), bits(host(g["sbar"])))
    X = synth.activations(wl, L.n, M, li)
    xq, sx, rs = ops.quant_act(cuda(X))
    Y1, _ = ops.linear(xq, sx, rs, 16, g["m"], g["sbar"], L.d, split=g["split"])
    Y2, _ = ops.linear_codes(xq, sx, gc["ucode"], st["wround"], st["z"], gc["zbar"], gc["sbar"], L.d)
    Y2h = host(Y2).view(np.uint16)
    assert np.array_equal(host(Y1).view(np.uint16), Y2h)
    rng = np.random.Generator(np.random.PCG64(31 + li))
    ts = rng.integers(0, M, 64)
    is_ = rng.integers(0, L.d, 64)
    m = oracle.merged_from_codes(ucode[is_], unpack4(host(st["wround"]))[is_], host(st["z"])[is_],
                                 host(gc["zbar"])[is_])
    mfull = np.zeros((L.d, L.n), np.int16)
    mfull[is_] = m
    _, y = oracle.linear_sampled(ts, is_, host(xq), host(sx), mfull, host(gc["sbar"]))
    assert np.array_equal(Y2h[ts, is_], y)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wl_index,li", [(3, 1), (3, 3), (4, 0), (1, 4)])
def test_merge_fused_full_size(ops, wl_index, li):
    """The fused single-pass MUL merge at full layer size equals the three-kernel merge
    (adaptation, row range, quantize) bit for bit on every output (FLUX out and mlp_out,
    Llama q, SD feed-forward)."""
    wl = synth.WORKLOADS[wl_index]
    L = wl.layers[li]
    lid = synth.layer_id(wl.index, li)
    seed = synth.PHILOX_SEED
    W = synth.weight(wl, li)
    A, Bm = synth.lora(wl, li)
    st = ops.setup_layer(cuda(W), wl.w_bits, seed, lid, synth.ALPHA)
    ubits = [b for mode, b in wl.modes if mode == "mul"][0]
    g = ops.merge_mul(st, cuda(A), cuda(Bm), wl.w_bits, ubits, seed, lid, dbg=True)
    f = ops.merge_mul_fused(st, cuda(A), cuda(Bm), wl.w_bits, ubits, seed, lid, dbg=True)
    for k in ("m", "uround", "zbar", "split"):
        assert torch.equal(g[k], f[k]), k
    assert np.array_equal(bits(host(g["sbar"])), bits(host(f["sbar"])))
    assert int(host(g["sat"])[0]) == int(host(f["sat"])[0])
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- every output
def check_layer_full(ops, wl, li, M):
    """Every output of one layer at its full size against the oracle run on the whole
    layer: set-up (c, W_round, z, s), the MUL merge (m, U_round, s_bar, z_bar, split
    codes, saturations; and the byte-plane storage with its plane codes) and the linear
    layer's bf16 outputs for all M tokens, from the int16 and the byte-plane storage."""
    L = wl.layers[li]
    lid = synth.layer_id(wl.index, li)
    W = synth.weight(wl, li)
    A, Bm = synth.lora(wl, li)
    X = synth.activations(wl, L.n, M, li)
    seed = synth.PHILOX_SEED
    mode, mbits = wl.modes[0]
    assert mode == "mul"
    print(f"full-output check: {wl.name} {L.name} {L.d}x{L.n} M={M}", flush=True)
    st = ops.setup_layer(cuda(W), wl.w_bits, seed, lid, synth.ALPHA)
    g = ops.merge_mul(st, cuda(A), cuda(Bm), wl.w_bits, mbits, seed, lid, dbg=True)
    gp = ops.merge_mul_planes(st, cuda(A), cuda(Bm), wl.w_bits, mbits, seed, lid)
    xq, sx, rs = ops.quant_act(cuda(X))
    Y, _ = ops.linear(xq, sx, rs, 16, g["m"], g["sbar"], L.d, split=g["split"])
    Yp, _ = ops.linear(xq, sx, rs, ops.B.INTLORA_W_INT16_PLANES, gp["planes"], gp["sbar"], L.d, split=gp["code"])
    ost = oracle.setup_layer(W, seed, lid, wl.w_bits, synth.ALPHA)
    gwr = host(st["wround"])
    gwr = unpack4(gwr) if wl.w_bits == 4 else gwr
    assert np.array_equal(bits(host(st["c"])), bits(ost["c"]))
    assert np.array_equal(gwr, ost["wround"])
    assert np.array_equal(host(st["z"]), ost["z"])
    assert np.array_equal(bits(host(st["s"])), bits(ost["s"]))
    ref = oracle.merge_mul(ost["wround"], ost["z"], ost["s"], ost["rstar"], A, Bm, mbits)
    lay, code = oracle.plane_store(ref["m"], ost["z"], ref["zbar"], wl.w_bits, mbits)
    del ost
    assert np.array_equal(host(gp["planes"]), lay)
    assert np.array_equal(host(gp["code"]), code)
    del lay
    assert np.array_equal(host(g["m"]), ref["m"])
    assert np.array_equal(host(g["uround"]), ref["uround"])
    assert np.array_equal(bits(host(g["sbar"])), bits(ref["sbar"]))
    assert np.array_equal(host(g["zbar"]), ref["zbar"])
    assert np.array_equal(host(g["split"]), oracle.plane_split(ref["m"]))
    assert int(host(g["sat"])[0]) == ref["sat"]
    oxq, osx, ors = oracle.quant_act(X)
    assert np.array_equal(host(xq), oxq)
    assert np.array_equal(bits(host(sx)), bits(osx))
    _, _, oy = oracle.linear(oxq, osx, ref["m"].astype(np.int32), ref["sbar"], want_exact=False)
    assert np.array_equal(host(Y).view(np.uint16), oy), (wl.name, L.name, M)
    assert np.array_equal(host(Yp).view(np.uint16), oy), (wl.name, L.name, M, "planes")
    del g, gp, st, Y, Yp, xq
    torch.cuda.empty_cache()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("li", [0, 1, 2, 3])
def test_flux_block_every_output(ops, li):
    """FLUX-like DiT block (W4A8, MUL U 4-bit, r = 32, 4608 tokens): each of the four
    layers in full."""
    wl = synth.WORKLOADS[3]
    check_layer_full(ops, wl, li, wl.tokens[0])


@pytest.mark.timeout(300)
def test_llama_gate_every_output(ops):
    """Llama-3-8B gate projection (14336 x 4096, W8A8, MUL U 8-bit, r = 64) at M = 2048,
    in full."""
    wl = synth.WORKLOADS[4]
    check_layer_full(ops, wl, 4, 2048)


def sweep_rows(d):
    """The sweep's row sample: every 64th row, and the last."""
    return np.array(sorted(set(range(0, d, 64)) | {d - 1}))


def check_sweep_block(ops, block, full):
    """The merge-only sweep of the Llama-shaped workload, transformer block `block`: all
    seven matrices merged on the GPU in full; the oracle checks every row (full) or the
    row sample (rows are independent: set-up and merge are row-local and R depends on
    (seed, layer, i, j) only)."""
    wl = synth.WORKLOADS[4]
    mode, mbits = wl.modes[0]
    seed = synth.PHILOX_SEED
    for li, L in enumerate(wl.layers):
        lid = synth.layer_id(wl.index, li, block)
        W = synth.sweep_weight(wl, li, block)
        A, Bm = synth.lora(wl, li, block=block)
        st = ops.setup_layer(cuda(W), wl.w_bits, seed, lid, synth.ALPHA)
        del W
        g = ops.merge_mul(st, cuda(A), cuda(Bm), wl.w_bits, mbits, seed, lid, dbg=True)
        rows = np.arange(L.d) if full else sweep_rows(L.d)
        Wr = synth.sweep_weight(wl, li, block, None if full else rows)
        c = oracle.vmc_scale(oracle.sigma_w(Wr), synth.ALPHA)
        if full:
            R = oracle.gen_r(L.d, L.n, seed, lid, c)
        else:
            R = np.concatenate([oracle.gen_r_rows(int(i), 1, L.n, seed, lid, c[k:k + 1]) for k, i in enumerate(rows)])
        wr, z, s = oracle.base_quant(Wr, R, wl.w_bits)
        ref = oracle.merge_mul(wr, z, s, R, A[rows], Bm, mbits)
        rt = torch.from_numpy(rows).cuda()
        pick = lambda t: t.index_select(0, rt).cpu().numpy()
        assert np.array_equal(bits(pick(st["c"])), bits(c)), (block, L.name)
        assert np.array_equal(pick(st["wround"]), wr)
        assert np.array_equal(pick(st["z"]), z)
        assert np.array_equal(bits(pick(st["s"])), bits(s))
        assert np.array_equal(pick(g["m"]), ref["m"]), (block, L.name)
        assert np.array_equal(pick(g["uround"]), ref["uround"])
        assert np.array_equal(bits(pick(g["sbar"])), bits(ref["sbar"]))
        assert np.array_equal(pick(g["zbar"]), ref["zbar"])
        assert np.array_equal(pick(g["split"]), oracle.plane_split(ref["m"]))
        if full:
            assert int(host(g["sat"])[0]) == ref["sat"]
        del g, st, R, ref
    torch.cuda.empty_cache()


@pytest.mark.timeout(300)
def test_llama_sweep_block0_every_row(ops):
    check_sweep_block(ops, 0, True)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("blocks", [(1, 11), (11, 21), (21, 32)])
def test_llama_sweep_blocks_row_sample(ops, blocks):
    for b in range(*blocks):
        print(f"sweep block {b}", flush=True)
        check_sweep_block(ops, b, False)
