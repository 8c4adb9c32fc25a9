"""Shared helpers of the GPU parity tests (not collected by pytest).

Parity protocol (tolerance tol: 1e-4 for fp32, 2e-2 for bf16/f16 storage;
the oracle runs in double on the same stored values):
  step check, teacher-forced (GPU and oracle get identical beams, hidden
  vectors and cumulative scores):
    - every beam's legal slots are exactly the oracle's legal tokens (sparse:
      slot j = j-th legal token; dense: slot = token), other slots -inf;
    - each legal log-prob within tol of the oracle's;
    - the GPU's picks: all candidates scoring above tau + tol are picked and
      none below tau - tol (tau = the oracle's K-th score), in non-increasing
      oracle order up to 2 tol; cum_out within tol; next rows bit-exact;
    - when the band |score - tau| <= tol holds only tau, the picks are the
      oracle's picks exactly.
  decode check: the GPU decode equals the GPU's own step-by-step trajectory,
  every step of which passes the step check; where the oracle's own decode
  meets no band ambiguity, the returned items are identical to the oracle's.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import sid_constrained_beam_amd as zgr  # noqa: E402
import workload  # noqa: E402

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_device_bits(bits, dtype):
    """Stored values (float32 array, or uint16 bit patterns) -> device tensor of dtype."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch_dtype(dtype))


class Setup:
    """One workload on the GPU and in the oracle."""

    def __init__(self, cfg, with_oracle=True, sids=None, slices="auto"):
        import torch
        self.cfg = cfg
        self.sids = workload.catalog(cfg) if sids is None else np.ascontiguousarray(sids, np.int32)
        fmt = cfg.fmt
        self.index, self.rank = zgr.zgr_index_upload(self.sids, cfg.V, fmt, slices=slices)
        self.W_bits, self.W_f32 = [], []
        for t in range(1, cfg.L + 1):
            b, f = workload.weights(cfg, t)
            self.W_bits.append(b)
            self.W_f32.append(f)
        self.W_dev = [to_device_bits(b, cfg.dtype) for b in self.W_bits]
        torch.cuda.synchronize()
        self.cat = oracle.Catalog(self.sids, cfg.V) if with_oracle else None
        self.stats = [self.index.stats(t) for t in range(1, cfg.L + 1)]
        self._decodes = {}

    def hidden_source(self, req_base=0, per_decode=0):
        """Hidden-vector callback: request ids req_base + i (advanced by
        per_decode at each new decode, for warm-up traffic)."""
        cfg = self.cfg
        state = {"base": req_base - per_decode}

        def fn(t, B, k_in, prefix_ptr, prefix_ld, hidden_ptr, stream_ptr):
            if t == 1:
                state["base"] += per_decode
            M = B * k_in
            prefix = np.empty((M, prefix_ld), np.int32)
            zgr.copy_to_host(prefix, prefix_ptr, stream_ptr)
            req = state["base"] + np.arange(M) // k_in
            bits, _ = workload.hidden(cfg, t, req, prefix, want_f32=False)
            zgr.copy_to_device(hidden_ptr, bits, stream_ptr)
            return 0
        return fn

    def plan(self, force=None, n_warmup=0, B=None, K=None, warm_base=None):
        cfg = self.cfg
        B = B or cfg.B
        K = K or cfg.K
        hs = None
        if n_warmup:
            hs = self.hidden_source(req_base=warm_base if warm_base is not None else B, per_decode=B)
        return zgr.zgr_plan_warmup(self.index, self.W_dev, cfg.dtype, cfg.d, B, K, hs, n_warmup,
                                   force)

    def oracle_decode(self, request, K=None, mode="filter_first"):
        cfg = self.cfg
        key = (request, K or cfg.K, mode)
        if key not in self._decodes:
            def hid(r, t, prefixes):
                return workload.hidden(cfg, t, np.full(len(prefixes), r, np.int64), prefixes)[1]
            self._decodes[key] = oracle.decode(self.cat, self.W_f32, hid, request, key[1],
                                               keep_steps=True, mode=mode)
        return self._decodes[key]


def run_gpu_step(setup, plan, t, prefixes, cum, B, K, requests, with_dbg=True, mode="filter_first"):
    """Run zgr_step on given beams.  prefixes [B*k_in, t-1] (rows of dead beams
    ignored), cum float32 [B*k_in] (-inf = dead).  Returns dict of numpy outputs
    and the inputs used.  In the unconstrained mode a live beam's row is 0."""
    import torch
    cfg = setup.cfg
    M = len(cum)
    k_in = M // B
    rows = np.full(M, -1, np.int32)
    for i in range(M):
        if np.isfinite(cum[i]):
            if mode == "unconstrained":
                rows[i] = 0
                continue
            rows[i] = setup.cat.node(prefixes[i, : t - 1]) if t > 1 else 0
            assert rows[i] >= 0
    req = np.repeat(np.asarray(requests, np.int64), k_in)
    pre = prefixes if t > 1 else np.zeros((M, 1), np.int32)
    bits, h32 = workload.hidden(cfg, t, req, np.ascontiguousarray(pre, np.int32))
    dev = dict(
        hidden=to_device_bits(bits, cfg.dtype),
        row_in=torch.from_numpy(rows).cuda(),
        cum_in=torch.from_numpy(np.asarray(cum, np.float32)).cuda(),
        parent=torch.empty(B * K, dtype=torch.int32, device="cuda"),
        token=torch.empty(B * K, dtype=torch.int32, device="cuda"),
        row_out=torch.empty(B * K, dtype=torch.int32, device="cuda"),
        cum_out=torch.empty(B * K, dtype=torch.float32, device="cuda"),
    )
    S = cfg.V if mode == "unconstrained" else setup.stats[t - 1]["stride"]
    dbg = torch.empty(M * S, dtype=torch.float32, device="cuda") if with_dbg is not False else None
    zgr.zgr_step(plan, t, dev["hidden"], dev["row_in"], dev["cum_in"], k_in, dev["parent"],
                 dev["token"], dev["row_out"], dev["cum_out"], dbg)
    zgr.zgr_plan_status(plan)
    out = {k: dev[k].cpu().numpy() for k in ("parent", "token", "row_out", "cum_out")}
    if with_dbg is True:
        out["dbg"] = dbg.cpu().numpy().reshape(M, S)
    elif with_dbg:
        # only the rows of the listed requests (full-size workloads)
        d2 = dbg.view(M, S)
        out["dbg"] = {q: d2[q * k_in:(q + 1) * k_in].cpu().numpy() for q in with_dbg}
    else:
        out["dbg"] = None
    out["h32"] = h32
    out["rows"] = rows
    return out


def check_step(setup, t, prefixes, cum, out, B, K, tol, check_dbg=True, requests=None,
               mode="filter_first", diag=None):
    """Step check against the oracle (in the same mode) on identical inputs
    (all requests, or the listed ones).  Returns the number of requests whose
    K-th score boundary was ambiguous.

    diag (a dict, optional) collects diagnostics beside the protocol, without
    loosening it: the largest |logp_gpu - logp_oracle| over the checked legal
    slots and |cum_out - oracle score| over the picks ("max_dlogp",
    "max_dscore"), and a second, tight selection check: with the band set to
    ten times the error this request-step actually shows (at least 8 ulps of
    the K-th score), a request whose K-th boundary is unambiguous at that band
    must pick exactly the oracle's candidates ("tight_exact" counts them,
    "tight_ambiguous" the others)."""
    cfg = setup.cfg
    M = len(cum)
    k_in = M // B
    st = setup.stats[t - 1]
    unc = mode == "unconstrained"
    dense = st["fmt"] != zgr.ZGR_FMT_SPARSE or unc  # slot = token
    ambiguous = 0
    for q in (range(B) if requests is None else requests):
        sl = slice(q * k_in, (q + 1) * k_in)
        pq = prefixes[sl, : t - 1] if t > 1 else np.zeros((k_in, 0), np.int32)
        cq = np.asarray(cum[sl], np.float64)
        res = setup.cat.step(t, setup.W_f32[t - 1], pq, cq, out["h32"][sl], K, mode)
        err_q = 0.0  # largest log-prob / score error seen in this request-step
        # (i) legal slots and their log-probs
        if check_dbg and out["dbg"] is not None:
            dbg = out["dbg"][q] if isinstance(out["dbg"], dict) else out["dbg"][sl]
            for k in range(k_in):
                m = res.cand_beam == k
                toks = res.cand_token[m]
                lp = res.cand_logp[m]
                row = dbg[k]
                legal_slots = toks if dense else np.arange(len(toks))
                got_legal = np.nonzero(np.isfinite(row))[0]
                assert np.array_equal(got_legal, np.sort(legal_slots)), (q, k, got_legal[:10], legal_slots[:10])
                err = np.abs(row[legal_slots] - lp)
                assert err.max(initial=0) <= tol, (q, k, err.max())
                err_q = max(err_q, float(err.max(initial=0)))
        # (ii) selection by the band protocol
        scores = {(int(b), int(v)): s for b, v, s in zip(res.cand_beam, res.cand_token, res.cand_score)}
        allv = np.sort(np.fromiter(scores.values(), np.float64))[::-1]
        kk = min(K, len(allv))
        o = slice(q * K, (q + 1) * K)
        par, tok, rowo, cumo = out["parent"][o], out["token"][o], out["row_out"][o], out["cum_out"][o]
        assert np.all(par[kk:] == -1) and np.all(tok[kk:] == -1) and np.all(rowo[kk:] == -1)
        assert np.all(np.isneginf(cumo[kk:]))
        if kk == 0:
            continue
        tau = allv[kk - 1]
        picks = []
        for i in range(kk):
            b = int(par[i]) - q * k_in
            assert 0 <= b < k_in, (q, i, par[i])
            key = (b, int(tok[i]))
            assert key in scores, ("illegal pick", q, key)
            s = scores[key]
            assert abs(cumo[i] - s) <= tol, (q, i, cumo[i], s)
            err_q = max(err_q, abs(float(cumo[i]) - s))
            if unc:
                assert rowo[i] == 0, (q, i)
            else:
                ext = np.concatenate([pq[b], [tok[i]]]).astype(np.int32)
                assert rowo[i] == setup.cat.node(ext), (q, i)
            picks.append(s)
        assert len(set(zip(par[:kk].tolist(), tok[:kk].tolist()))) == kk
        picks = np.array(picks)
        above = sum(1 for s in scores.values() if s > tau + tol)
        assert np.sum(picks > tau + tol) == above
        assert np.all(picks >= tau - tol)
        assert np.all(np.diff(picks) <= 2 * tol)
        band = sum(1 for s in scores.values() if abs(s - tau) <= tol)
        want = list(zip(res.sel_beam.tolist(), res.sel_token.tolist()))
        got = [(int(par[i]) - q * k_in, int(tok[i])) for i in range(kk)]
        if band == 1:
            assert set(got) == set(want), (q, "selection differs without ambiguity")
        else:
            ambiguous += 1
        if diag is not None:
            diag["max_dlogp"] = max(diag.get("max_dlogp", 0.0), err_q if check_dbg else 0.0)
            diag["max_dscore"] = max(diag.get("max_dscore", 0.0),
                                     max(abs(float(cumo[i]) - scores[g]) for i, g in enumerate(got)))
            tight = max(10.0 * err_q, 8.0 * float(np.spacing(np.float32(abs(tau)))))
            diag["tight_band_max"] = max(diag.get("tight_band_max", 0.0), tight)
            if len(allv) > kk and allv[kk - 1] - allv[kk] <= tight:
                diag["tight_ambiguous"] = diag.get("tight_ambiguous", 0) + 1
            else:
                assert set(got) == set(want), (q, "selection differs at ten times the observed error")
                diag["tight_exact"] = diag.get("tight_exact", 0) + 1
    return ambiguous


def gpu_trajectory(s, plan, requests, mode="filter_first"):
    """The GPU's own step-by-step decode; every step checked against the oracle
    on the GPU's beams.  Returns final (rows, sids, scores) and ambiguity count."""
    cfg = s.cfg
    B, K, L = cfg.B, cfg.K, cfg.L
    tol = TOL[cfg.dtype]
    prefixes = np.zeros((B, 0), np.int32)
    cum = np.zeros(B, np.float32)
    amb = 0
    out = None
    for t in range(1, L + 1):
        out = run_gpu_step(s, plan, t, prefixes, cum, B, K, requests, mode=mode)
        amb += check_step(s, t, prefixes, cum, out, B, K, tol, mode=mode)
        par = out["parent"]
        new = np.full((B * K, t), -1, np.int32)
        ok = par >= 0
        if t > 1:
            new[ok, : t - 1] = prefixes[par[ok]]
        new[ok, t - 1] = out["token"][ok]
        prefixes, cum = new, out["cum_out"]
    return out["row_out"].reshape(B, K), prefixes.reshape(B, K, L), cum.reshape(B, K), amb


def assert_same_ranking(got, want, want_score, tol, what=""):
    """End-to-end comparison of a returned list with the oracle's (keys are
    item ids, or SIDs where off-catalog codes share the id -1).  The lists
    hold the same entries, and position i holds an entry whose oracle score
    is within tol of the oracle's i-th score: entries whose oracle scores
    differ by less than the tolerance may come in either order (a float32
    path cannot order scores closer than its own rounding; the step check
    allows the same band), every other pair keeps the oracle's order."""
    got = [tuple(np.atleast_1d(x).tolist()) for x in got]
    want = [tuple(np.atleast_1d(x).tolist()) for x in want]
    assert sorted(got) == sorted(want), (what, "different entries")
    score = {}
    for w, s in zip(want, want_score):
        score.setdefault(w, s)
    for i, g in enumerate(got):
        a, b = score[g], want_score[i]
        assert (a == b) or abs(a - b) <= tol, (what, i, g, a, b)


def oracle_unambiguous(dec, K, tol):
    for st in dec.steps:
        sc = np.sort(st["res"].cand_score)[::-1]
        if len(sc) > K:
            tau = sc[K - 1]
            if np.sum(np.abs(sc - tau) <= tol) > 1:
                return False
    return True
