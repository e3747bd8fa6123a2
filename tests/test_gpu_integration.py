"""Integration identity: a toy decoder built only from the C ABI plus host glue.  QSPEC greedy
decoding (gamma W4A4 draft steps writing low-precision KV, one W4A16 verify pass over gamma + 1
positions, greedy acceptance, KV overwrite of the committed positions) must emit exactly the
token stream of plain W4A16 greedy decoding.  (QSPEC notes, QSPEC structure: the W4A4 draft and
the W4A16 verifier share one set of 4-bit weights, verification keeps the output W4A16-equivalent
and the verifier's KV replaces the draft's for accepted tokens; speculative-decoding background:
greedy acceptance and the first-reject cutoff.)

The toy model: an embedding table E [V][H]; a one-projection "KV" row kv(t) = W_kv E[token_t]
cached per position; next-token logits = lm_head(E[token_t] + mean of the cached rows 0..t).
The identity holds because row results of qspec_gemm_w4a16 do not depend on M within a batch
tier (M = 1 in plain decoding, gamma + 1 in verification), so the verifier reproduces plain
decoding's KV rows and logits bit for bit.

A second toy replaces the mean with qspec_attention over the shared cache (queries E[token],
keys = values = the cached rows); there the identity also needs every query row of an attention
call to be bit-identical whether it is computed alone (Q = 1) or with gamma others (Q = gamma + 1)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_speculative_decoding_amd as q
import synthetic_inputs as si
from gpu_helpers import DEV, bf16_dev, cu, note, weights_dev

pytestmark = pytest.mark.gpu

V, H, HEADS, D, CTX = 1024, 256, 2, 128, 96


class Toy:
    def __init__(self, seed: int, unrelated_draft_head: bool = False):
        self.E = si.activations(V, H, seed=seed)                  # bf16 bits [V][H]
        self.Ef = self.E.astype(np.uint32) << 16
        self.Ef = self.Ef.view(np.float32)
        self.w_kv = weights_dev(si.weights(H, H, seed=seed + 1))
        self.w_lm = weights_dev(si.weights(H, V, seed=seed + 2))
        # a draft head unrelated to the target's: most drafts are rejected, which exercises the
        # correction token and the overwrite of rejected draft KV on every round
        self.w_lm_draft = weights_dev(si.weights(H, V, seed=seed + 3)) if unrelated_draft_head else self.w_lm

    # ---- glue (host): h = bf16(E[token] + mean of the KV rows), the same arithmetic everywhere
    def hidden(self, tok: int, rows: np.ndarray) -> np.ndarray:
        kv = (rows.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        mean = kv.sum(axis=0) / kv.shape[0]
        return si.f32_to_bf16_bits((self.Ef[tok].astype(np.float64) + mean).astype(np.float32))

    # ---- W4A16 (verify precision)
    def kv16(self, toks) -> np.ndarray:
        x = bf16_dev(self.E[np.asarray(toks)])
        y = torch.empty((len(toks), H), dtype=torch.bfloat16, device=DEV)
        q.qspec_gemm_w4a16(x, *self.w_kv, y)
        return y.view(torch.int16).cpu().numpy().view(np.uint16)

    def logits16(self, hs: np.ndarray) -> torch.Tensor:
        y = torch.empty((hs.shape[0], V), dtype=torch.float32, device=DEV)
        q.qspec_gemm_w4a16(bf16_dev(hs), *self.w_lm, y)
        return y

    # ---- W4A4 (draft precision): quantize, then the draft layer
    def _w4a4(self, x_bits: np.ndarray, w, N: int, out) -> torch.Tensor:
        M = x_bits.shape[0]
        codes = torch.empty((M, H // 2), dtype=torch.uint8, device=DEV)
        scales = torch.empty((M, H // 128), dtype=torch.float32, device=DEV)
        q.qspec_quantize_act(bf16_dev(x_bits), codes, scales)
        y = torch.empty((M, N), dtype=out, device=DEV)
        q.qspec_gemm_w4a4(codes, scales, *w, y)
        return y

    def kv4(self, tok: int) -> np.ndarray:
        y = self._w4a4(self.E[[tok]], self.w_kv, H, torch.bfloat16)
        return y.view(torch.int16).cpu().numpy().view(np.uint16)[0]

    def logits4(self, h: np.ndarray) -> np.ndarray:
        return self._w4a4(h[None], self.w_lm_draft, V, torch.float32).cpu().numpy()[0]


def plain_greedy(m: Toy, first: int, n: int) -> list:
    toks, rows = [first], []
    while len(toks) < n + 1:
        t = len(toks) - 1
        rows.append(m.kv16([toks[t]])[0])
        h = m.hidden(toks[t], np.stack(rows))
        toks.append(int(np.argmax(m.logits16(h[None]).cpu().numpy()[0])))
    return toks


def qspec_greedy(m: Toy, first: int, n: int, gamma: int):
    cache = torch.zeros((1, 1, 2, HEADS, CTX, D), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((q.qspec_verify_workspace_bytes(q.QSPEC_GREEDY, 1, gamma, V),), dtype=torch.uint8, device=DEV)
    acc = torch.zeros((1,), dtype=torch.int32, device=DEV)
    out = torch.zeros((1, gamma + 1), dtype=torch.int32, device=DEV)

    def rows(lo, hi):   # cached KV rows lo..hi-1 (slot 0), [n][H] bf16 bits
        r = cache[0, 0, 0, :, lo:hi, :].permute(1, 0, 2).reshape(hi - lo, H)
        return r.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    toks, p, accepts = [first], 0, []
    while len(toks) < n + 1:
        # draft: gamma W4A4 steps, each writing its low-precision KV row at its position
        d, tok = [], toks[p]
        for j in range(gamma):
            kvd = torch.from_numpy(m.kv4(tok).view(np.int16)).view(torch.bfloat16).to(DEV)
            cache[0, 0, 0, :, p + j, :] = kvd.view(HEADS, D)
            h = m.hidden(tok, rows(0, p + j + 1))
            tok = int(np.argmax(m.logits4(h)))
            d.append(tok)
        # verify: one W4A16 pass over positions p .. p + gamma
        vt = [toks[p]] + d                                         # tokens at p .. p + gamma
        vkv = m.kv16(vt)                                           # [gamma + 1][H]
        base = rows(0, p)
        hs = np.stack([m.hidden(vt[j], np.concatenate([base, vkv[: j + 1]])) for j in range(gamma + 1)])
        target = m.logits16(hs).view(1, gamma + 1, V)
        q.qspec_verify_accept(q.QSPEC_GREEDY, target, None, cu(np.array([d], np.int32)), None, None, acc, out, ws)
        stage = torch.zeros((1, 1, 2, HEADS, gamma + 1, D), dtype=torch.bfloat16, device=DEV)
        stage[0, 0, 0] = torch.from_numpy(vkv.view(np.int16)).view(torch.bfloat16).to(DEV).view(
            gamma + 1, HEADS, D).permute(1, 0, 2)
        q.qspec_kv_overwrite(cache, stage, cu(np.array([p], np.int32)), acc)
        A = int(acc.cpu()[0])
        committed = out.cpu().numpy()[0, : A + 1].tolist()
        assert committed[:A] == d[:A]
        accepts.append(A)
        toks.extend(committed)
        p += A + 1
    return toks[: n + 1], accepts


@pytest.mark.parametrize("seed,gamma,unrelated", [(11, 4, False), (23, 2, False), (37, 7, False), (5, 4, True)])
def test_qspec_greedy_loop_equals_plain_w4a16_greedy(seed, gamma, unrelated):
    note(f"toy decoder identity seed={seed} gamma={gamma} unrelated draft head={unrelated}")
    m = Toy(seed, unrelated)
    n = 40
    ref = plain_greedy(m, first=seed % V, n=n)
    got, accepts = qspec_greedy(m, first=seed % V, n=n, gamma=gamma)
    note(f"accept counts per round: {accepts}")
    assert got == ref
    assert len(accepts) > 1
    if unrelated:
        assert accepts.count(0) > len(accepts) // 2       # mostly first-position rejections
    else:
        assert sum(accepts) > 0                           # the drafts were used


# ---- the same identity with attention over the shared cache -------------------------------------
# hidden(t) = bf16(E[token_t] + attention(q = E[token_t], keys = values = the cached KV rows 0..t)),
# through qspec_attention: Q = 1 per plain step and per draft step (over a cache holding the
# draft's W4A4 rows for the current round), Q = gamma + 1 for the verify pass (over the committed
# rows plus the verifier's gamma + 1 staged rows); qspec_kv_overwrite then commits A + 1 rows.

class AttnToy(Toy):
    def attend(self, cache, toks, pos):
        """toks: the Q query tokens at positions pos .. pos + Q - 1; returns hidden bf16 bits [Q][H]."""
        Qn = len(toks)
        qd = bf16_dev(self.E[np.asarray(toks)]).view(1, Qn, HEADS, D)
        out = torch.empty((1, Qn, HEADS, D), dtype=torch.bfloat16, device=DEV)
        ws = torch.empty((q.qspec_attention_workspace_bytes(1, Qn, HEADS, HEADS, CTX),), dtype=torch.uint8, device=DEV)
        q.qspec_attention(qd, cache[0], cu(np.array([pos], np.int32)), D ** -0.5, out, ws)
        o = (out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(Qn, H).astype(np.uint32) << 16).view(np.float32)
        return si.f32_to_bf16_bits(self.Ef[np.asarray(toks)] + o)


def write_row(cache, t, bits):
    row = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV).view(HEADS, D)
    cache[0, 0, 0, :, t, :] = row                  # key
    cache[0, 0, 1, :, t, :] = row                  # value


def plain_greedy_attn(m: AttnToy, first: int, n: int) -> list:
    cache = torch.zeros((1, 1, 2, HEADS, CTX, D), dtype=torch.bfloat16, device=DEV)
    toks = [first]
    while len(toks) < n + 1:
        t = len(toks) - 1
        write_row(cache, t, m.kv16([toks[t]])[0])
        h = m.attend(cache, [toks[t]], t)
        toks.append(int(np.argmax(m.logits16(h).cpu().numpy()[0])))
    return toks


def qspec_greedy_attn(m: AttnToy, first: int, n: int, gamma: int):
    cache = torch.zeros((1, 1, 2, HEADS, CTX, D), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((q.qspec_verify_workspace_bytes(q.QSPEC_GREEDY, 1, gamma, V),), dtype=torch.uint8, device=DEV)
    acc = torch.zeros((1,), dtype=torch.int32, device=DEV)
    out = torch.zeros((1, gamma + 1), dtype=torch.int32, device=DEV)
    toks, p, accepts = [first], 0, []
    while len(toks) < n + 1:
        d, tok = [], toks[p]
        for j in range(gamma):                                     # draft: W4A4 KV row, Q = 1 attention
            write_row(cache, p + j, m.kv4(tok))
            tok = int(np.argmax(m.logits4(m.attend(cache, [tok], p + j)[0])))
            d.append(tok)
        vt = [toks[p]] + d
        vkv = m.kv16(vt)                                           # the verifier's rows for p .. p + gamma
        vcache = cache.clone()
        for j in range(gamma + 1):
            write_row(vcache, p + j, vkv[j])
        target = m.logits16(m.attend(vcache, vt, p)).view(1, gamma + 1, V)
        q.qspec_verify_accept(q.QSPEC_GREEDY, target, None, cu(np.array([d], np.int32)), None, None, acc, out, ws)
        stage = torch.zeros((1, 1, 2, HEADS, gamma + 1, D), dtype=torch.bfloat16, device=DEV)
        rows = torch.from_numpy(vkv.view(np.int16)).view(torch.bfloat16).to(DEV).view(gamma + 1, HEADS, D)
        stage[0, 0, 0] = rows.permute(1, 0, 2)
        stage[0, 0, 1] = rows.permute(1, 0, 2)
        q.qspec_kv_overwrite(cache, stage, cu(np.array([p], np.int32)), acc)
        A = int(acc.cpu()[0])
        committed = out.cpu().numpy()[0, : A + 1].tolist()
        assert committed[:A] == d[:A]
        # the committed positions now hold exactly the verifier's rows
        assert torch.equal(cache[0, 0, :, :, p:p + A + 1, :], vcache[0, 0, :, :, p:p + A + 1, :])
        accepts.append(A)
        toks.extend(committed)
        p += A + 1
    return toks[: n + 1], accepts


@pytest.mark.parametrize("seed,gamma,unrelated", [(11, 4, False), (29, 3, False), (5, 4, True)])
def test_qspec_greedy_with_attention_over_the_shared_cache_equals_plain_greedy(seed, gamma, unrelated):
    note(f"toy decoder with attention seed={seed} gamma={gamma} unrelated draft head={unrelated}")
    m = AttnToy(seed, unrelated)
    n = 40
    ref = plain_greedy_attn(m, first=seed % V, n=n)
    got, accepts = qspec_greedy_attn(m, first=seed % V, n=n, gamma=gamma)
    note(f"accept counts per round: {accepts}")
    assert got == ref
    assert len(accepts) > 1
    if not unrelated:
        assert sum(accepts) > 0


# ---- the identity with a batch of sequences, across W4A16 batch tiers ------------------------
# Plain decoding of B sequences runs the W4A16 layers at M = B; QSPEC verification at
# M = B (gamma + 1).  With the vocabulary head at V2 = 16384 columns (its decode tier ends at
# M = 20) and the KV projection at 256 x 256 (decode tier up to M = 32), B = 4 with gamma = 5
# verifies the head at M = 24 and B = 16 verifies both layers at M = 80 -- in a different tier
# from plain decoding.  Rows then agree to fp32 rounding instead of bit for bit, so the committed
# tokens may differ from plain decoding only where plain decoding's own choice is a near tie: a
# token may differ only where the oracle's top-2 logit gap of the plain run's hidden state is
# below 1e-4 of the top logit.  B = 1 with gamma = 16 verifies at M = 17, inside the decode tier
# of both layers: the same reduction order as plain decoding, so the tokens are equal outright.

V2 = 16384


class BatchToy(Toy):
    def __init__(self, seed: int):
        self.E = si.activations(V2, H, seed=seed)
        self.Ef = (self.E.astype(np.uint32) << 16).view(np.float32)
        self.w_kv = weights_dev(si.weights(H, H, seed=seed + 1))
        self.w_lm_host = si.weights(H, V2, seed=seed + 2)
        self.w_lm = weights_dev(self.w_lm_host)
        self.w_lm_draft = self.w_lm

    def logits16_rows(self, hs: np.ndarray) -> np.ndarray:
        y = torch.empty((hs.shape[0], V2), dtype=torch.float32, device=DEV)
        q.qspec_gemm_w4a16(bf16_dev(hs), *self.w_lm, y)
        return y

    def kv4_rows(self, toks) -> np.ndarray:
        y = self._w4a4(self.E[np.asarray(toks)], self.w_kv, H, torch.bfloat16)
        return y.view(torch.int16).cpu().numpy().view(np.uint16)

    def logits4_rows(self, hs: np.ndarray) -> np.ndarray:
        return self._w4a4(hs, self.w_lm_draft, V2, torch.float32).cpu().numpy()


def plain_greedy_batch(m: BatchToy, firsts, n: int):
    B = len(firsts)
    toks = [[f] for f in firsts]
    rows = [[] for _ in range(B)]
    hidden = [[] for _ in range(B)]           # hidden state behind each emitted token
    for t in range(n):
        kv = m.kv16([toks[b][t] for b in range(B)])              # M = B
        hs = []
        for b in range(B):
            rows[b].append(kv[b])
            hs.append(m.hidden(toks[b][t], np.stack(rows[b])))
        hs = np.stack(hs)
        nxt = np.argmax(m.logits16_rows(hs).cpu().numpy(), axis=1)   # M = B
        for b in range(B):
            toks[b].append(int(nxt[b]))
            hidden[b].append(hs[b])
    return toks, hidden


def qspec_greedy_batch(m: BatchToy, firsts, n: int, gamma: int):
    B = len(firsts)
    ctx = (n + 1) * (gamma + 1) + gamma + 1      # a sequence ahead of the slowest keeps drafting
    cache = torch.zeros((1, B, 2, HEADS, ctx, D), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty((q.qspec_verify_workspace_bytes(q.QSPEC_GREEDY, B, gamma, V2),), dtype=torch.uint8, device=DEV)
    acc = torch.zeros((B,), dtype=torch.int32, device=DEV)
    out = torch.zeros((B, gamma + 1), dtype=torch.int32, device=DEV)

    def rows(b, lo, hi):
        r = cache[0, b, 0, :, lo:hi, :].permute(1, 0, 2).reshape(hi - lo, H)
        return r.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    toks = [[f] for f in firsts]
    p = [0] * B
    accepts = []
    while min(len(t) for t in toks) < n + 1:
        cur = [toks[b][p[b]] for b in range(B)]
        d = [[] for _ in range(B)]
        for j in range(gamma):                                   # draft steps at M = B
            kvd = m.kv4_rows(cur)
            hs = []
            for b in range(B):
                cache[0, b, 0, :, p[b] + j, :] = torch.from_numpy(kvd[b].view(np.int16)).view(
                    torch.bfloat16).to(DEV).view(HEADS, D)
                hs.append(m.hidden(cur[b], rows(b, 0, p[b] + j + 1)))
            nxt = np.argmax(m.logits4_rows(np.stack(hs)), axis=1)
            for b in range(B):
                d[b].append(int(nxt[b]))
                cur[b] = int(nxt[b])
        vt = [[toks[b][p[b]]] + d[b] for b in range(B)]
        vkv = m.kv16([t for b in range(B) for t in vt[b]]).reshape(B, gamma + 1, H)   # M = B (gamma + 1)
        hs = np.stack([m.hidden(vt[b][j], np.concatenate([rows(b, 0, p[b]), vkv[b, : j + 1]]))
                       for b in range(B) for j in range(gamma + 1)])
        target = m.logits16_rows(hs).view(B, gamma + 1, V2)                            # M = B (gamma + 1)
        q.qspec_verify_accept(q.QSPEC_GREEDY, target, None, cu(np.array(d, np.int32)), None, None, acc, out, ws)
        stage = torch.zeros((1, B, 2, HEADS, gamma + 1, D), dtype=torch.bfloat16, device=DEV)
        stage[0, :, 0] = torch.from_numpy(vkv.view(np.int16)).view(torch.bfloat16).to(DEV).view(
            B, gamma + 1, HEADS, D).permute(0, 2, 1, 3)
        q.qspec_kv_overwrite(cache, stage, cu(np.array(p, np.int32)), acc)
        A = acc.cpu().numpy()
        o = out.cpu().numpy()
        for b in range(B):
            committed = o[b, : A[b] + 1].tolist()
            assert committed[: A[b]] == d[b][: A[b]]
            toks[b].extend(committed)
            p[b] += int(A[b]) + 1
        accepts.append(A.tolist())
    return [t[: n + 1] for t in toks], accepts


@pytest.mark.parametrize("B,gamma", [(4, 5), (16, 4), (1, 16)])
def test_qspec_greedy_batch_equals_plain_w4a16_greedy_across_tiers(B, gamma):
    note(f"toy decoder identity across W4A16 tiers B={B} gamma={gamma}")
    m = BatchToy(seed=41 + B)
    plain_tier = q.qspec_gemm_w4a16_tier(B, H, V2)
    verify_tier = q.qspec_gemm_w4a16_tier(B * (gamma + 1), H, V2)
    cross = plain_tier[0] != verify_tier[0]
    assert cross == (B > 1)                                # B > 1: the head is verified in another tier
    n = 24 if B == 16 else 32
    firsts = [(97 * b + 5) % V2 for b in range(B)]
    ref, hid = plain_greedy_batch(m, firsts, n)
    got, accepts = qspec_greedy_batch(m, firsts, n, gamma)
    note(f"accept counts per round: {accepts}")
    assert sum(sum(a) for a in accepts) > 0
    flips = 0
    for b in range(B):
        if got[b] == ref[b]:
            continue
        assert cross, (b, got[b], ref[b])                  # one tier: one reduction order, no flips
        i = next(k for k in range(n + 1) if got[b][k] != ref[b][k])
        h = hid[b][i - 1]                                   # plain run's hidden state before token i
        logits = oracle.gemm_w4a16(h[None], m.w_lm_host["codes"], m.w_lm_host["meta"])[0]
        top2 = np.sort(logits)[-2:]
        gap = top2[1] - top2[0]
        assert gap < 1e-4 * abs(top2[1]), (b, i, gap, top2)
        flips += 1
    note(f"sequences with a near-tie flip: {flips} of {B}")
