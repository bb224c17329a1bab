"""GPU parity of branching: restore to an earlier position and fork one sequence into others.

Each case keeps, per sequence, the token stream the state should now hold (a host simulation of
the window counts decides which entries a restore can drop), runs the fp64 oracle on exactly that
stream and compares every later replay output and the final state. Forks run both ways: copying
the checkpoint, and sharing it (the copies read the source's checkpoint slot and move to a slot
of their own at the next fold). A fork is also checked bit for bit: right after it the
destination's buffered entries and pointers equal the source's (and, when copied, its checkpoint
bytes), untouched sequences keep theirs, and a copy fed the source's inputs reproduces the
source's outputs. With shared checkpoints every fold launch must leave each sequence on one of
its own two slots with no slot read twice.
"""
import numpy as np
import pytest
import torch

import oracle
from harness import assert_close, sample_pairs, to_dev
from ssm_decode_state_amd import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
bd = pytest.importorskip("ssm_decode_state_amd.binding")
DEV = torch.device("cuda:0")

GDN_KEYS = ("q", "k", "v", "beta", "g")


class Branches:
    """One state on the GPU plus the host record of what each sequence holds."""

    def __init__(self, shape, seed, h0_std, rc=0, scale=1.0, share=0):
        self.shape, self.seed, self.scale = shape, seed, scale
        self.m2 = shape.kind == synth.MAMBA2
        self.A, self.D = synth.head_constants(shape, seed)
        self.h0 = synth.initial_state(shape, seed, h0_std) if h0_std else None
        cfg = bd.make_config(shape.kind, shape.batch, shape.heads, shape.groups, shape.dim_p,
                             shape.dim_n, shape.window, shape.max_draft,
                             bd.SSM_IN_BF16 if shape.in_bf16 else bd.SSM_IN_F32, rc, scale, share)
        self.st = bd.State(cfg, None if self.h0 is None else self.h0.to(DEV),
                           None if self.A is None else self.A.to(DEV),
                           None if self.D is None else self.D.to(DEV))
        self.steps = []
        self.stream = [[] for _ in range(shape.batch)]  # (step, batch row) of every held entry
        self.count = [0] * shape.batch                   # entries since the last fold
        self.counts_known = True                          # false once shared folds make them vary
        self.origin = list(range(shape.batch))            # whose initial state a sequence holds
        self.got = {}                                     # (b, h) -> [(stream position, y)]
        self.y = torch.empty(shape.batch, shape.heads, shape.dim_p, device=DEV)

    def decode(self, pairs, inputs=None):
        t = len(self.steps)
        d = inputs if inputs is not None else synth.token_inputs(self.shape, self.seed, "branch", t)
        self.steps.append(d)
        bd.ssm_replay_decode(self.st, to_dev(d, DEV), self.y)
        for b in range(self.shape.batch):
            self.stream[b].append((t, b))
            self.count[b] += 1
            if self.count[b] == self.shape.window:
                self.count[b] = 0
        if pairs:
            bi = torch.tensor([b for (b, _) in pairs], device=DEV)
            hi = torch.tensor([h for (_, h) in pairs], device=DEV)
            ys = self.y[bi, hi].cpu().double().numpy()
            for i, (b, h) in enumerate(pairs):
                self.got.setdefault((b, h), []).append((len(self.stream[b]) - 1, ys[i]))

    def spec(self, S, acc, pairs):
        """One speculative round of S drafts; sequence b keeps its first acc[b] drafts."""
        t = len(self.steps)
        d = synth.token_inputs(self.shape, self.seed, "branch-spec", t, ntok=S)
        for j in range(S):
            self.steps.append({k: v[:, j:j + 1] for k, v in d.items()})
        sh = self.shape
        y = torch.empty(sh.batch, S, sh.heads, sh.dim_p, device=DEV)
        bd.ssm_spec_append(self.st, S, to_dev(d, DEV), y)
        bd.ssm_spec_rollback(self.st, torch.tensor(acc, dtype=torch.int32, device=DEV))
        ys = y.cpu().double().numpy()
        for (b, h) in pairs:
            for j in range(acc[b]):
                self.got.setdefault((b, h), []).append((len(self.stream[b]) + j, ys[b, j, h]))
        for b in range(sh.batch):
            self.stream[b] += [(t + j, b) for j in range(acc[b])]
        self.counts_known = False  # the folds after a rollback are decided on the device

    def restore(self, n_back):
        assert self.counts_known
        bd.ssm_restore(self.st, torch.tensor(n_back, dtype=torch.int32, device=DEV))
        for b, n in enumerate(n_back):
            n = max(0, min(n, self.count[b]))
            if n:
                del self.stream[b][-n:]
            self.count[b] -= n
            keep = len(self.stream[b])  # outputs of dropped positions belong to the old stream
            for key in [k for k in self.got if k[0] == b]:
                self.got[key] = [(p, y) for (p, y) in self.got[key] if p < keep]

    def fork(self, src, dst):
        bd.ssm_fork(self.st, src, dst)
        for s, d in zip(src, dst):
            self.stream[d] = list(self.stream[s])
            self.count[d] = self.count[s]
            self.origin[d] = self.origin[s]
            for key in [k for k in self.got if k[0] == d]:
                del self.got[key]  # outputs from before the fork belong to the old stream

    def oracle_pair(self, b, h):
        """fp64 outputs over the stream sequence b holds, and its final state, for head h."""
        sh = self.shape
        hg = h // (sh.heads // sh.groups)
        ent, o = self.stream[b], self.origin[b]

        def col(key, hh):
            return synth.to_f64(torch.stack([self.steps[t][key][r, 0, hh] for (t, r) in ent]))[None]

        if self.m2:
            h0 = None if self.h0 is None else self.h0[o, h].double().numpy()[None]
            y, hT, _ = oracle.m2_sequential(self.A.double().numpy()[[h]],
                                            self.D.double().numpy()[[h]], h0, col("x", h),
                                            col("B", hg), col("C", hg), col("dt", h))
        else:
            S0 = None if self.h0 is None else self.h0[o, h].double().numpy()[None]
            fn = oracle.kda_sequential if sh.kind == synth.KDA else oracle.gdn_sequential
            y, hT, _ = fn(S0, *[col(k, h) for k in GDN_KEYS], scale=self.scale)
        return y[0], hT[0]

    def slots(self):
        """(checkpoint slot of every head [B][H], reader count of every slot)."""
        c, L = self.st.cfg, self.st.layout
        p = self.st.region(L.off_ptr, c.batch * c.heads * 16).view(torch.int32).view(c.batch, c.heads, 4)
        rc = self.st.region(L.off_refcnt, L.ckpt_slots * 4).view(torch.int32)
        return p[..., 2].cpu(), rc.cpu()

    def check_slots_after_fold(self):
        """After a fold launch nobody shares: every sequence is on one of its own slots and the
        reader counts are exact."""
        torch.cuda.synchronize()
        slot, rc = self.slots()
        B = self.shape.batch
        assert torch.all(slot == slot[:, :1]), "the heads of a sequence disagree on its slot"
        s0 = slot[:, 0]
        own = (s0 == torch.arange(B)) | (s0 == torch.arange(B) + B)
        assert bool(own.all()), "a sequence still reads a slot it does not own: %s" % s0.tolist()
        assert torch.equal(rc, torch.bincount(s0.long(), minlength=rc.numel()).int())

    def check(self, pairs, what):
        bd.ssm_flush(self.st, bd.SSM_FLUSH_ALL)
        if self.st.cfg.share_ckpt:
            self.check_slots_after_fold()
        sh = self.shape
        nat = torch.empty(sh.batch, sh.heads, sh.dim_p, sh.dim_n, device=DEV)
        bd.ssm_ckpt_export(self.st, nat)
        torch.cuda.synchronize()
        for (b, h) in pairs:
            oy, oT = self.oracle_pair(b, h)
            rec = self.got.get((b, h), [])
            if rec:
                gy = np.stack([y for (_, y) in rec])
                assert_close(gy, oy[[p for (p, _) in rec]], (-1,), "%s outputs (%d, %d)" % (what, b, h))
            assert_close(nat[b, h].cpu().double().numpy(), oT, (-2, -1),
                         "%s final state (%d, %d)" % (what, b, h))


def _shape(kind, B, H, L=8, bf16=True, S=1):
    if kind == synth.MAMBA2:
        return synth.Shape(kind, B, H, 1, 64, 128, L, S, in_bf16=bf16)
    return synth.Shape(kind, B, H, H, 128, 64, L, S, in_bf16=bf16)


KINDS = [synth.MAMBA2, synth.GDN, synth.KDA]


@pytest.mark.parametrize("share", [0, 1])
@pytest.mark.parametrize("kind", KINDS)
def test_restore_then_decode(kind, share):
    B, H = 5, 2
    br = Branches(_shape(kind, B, H), 300 + kind, 0.3, scale=0.7 if kind else 1.0, share=share)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    for _ in range(13):  # one fold, then five entries buffered
        br.decode(pairs)
    br.restore([2, 0, 9, -3, 5])  # 9 is clamped to the five buffered entries
    for _ in range(6):
        br.decode(pairs)
    br.restore([1, 3, 0, 7, 2])
    br.restore([1, 0, 0, 0, 0])  # two restores in a row
    for _ in range(9):  # every sequence folds again
        br.decode(pairs)
    br.check(pairs, "restore")


def test_restore_after_fold_drops_nothing():
    br = Branches(_shape(synth.MAMBA2, 2, 2, L=4), 311, 0.3)
    pairs = [(0, 0), (1, 1)]
    for _ in range(8):  # both windows just folded
        br.decode(pairs)
    br.restore([4, 1])
    for _ in range(3):
        br.decode(pairs)
    br.check(pairs, "restore after a fold")


@pytest.mark.parametrize("share", [0, 1])
@pytest.mark.parametrize("kind", KINDS)
def test_fork_then_decode(kind, share):
    B, H = 6, 2
    br = Branches(_shape(kind, B, H), 320 + kind, 0.3, share=share)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    for _ in range(11):
        br.decode(pairs)
    br.fork([0, 0, 1], [3, 4, 5])  # one prefix into two continuations, and a plain copy
    for _ in range(2):
        br.decode(pairs)
    br.fork([3, 2], [1, 0])        # sources that read a shared slot, and a sharer overwritten
    for _ in range(8):
        br.decode(pairs)
    if share:
        br.check_slots_after_fold()  # the window closed: every sharer moved
    br.restore([0, 2, 0, 1, 3, 0])  # a restore on forked sequences
    for _ in range(4):
        br.decode(pairs)
    br.check(pairs, "fork")


@pytest.mark.parametrize("share", [0, 1])
@pytest.mark.parametrize("kind", KINDS)
def test_fork_then_speculative_rounds(kind, share):
    # after a rollback the fold is a device predicate: sharers with fewer than L entries must
    # still move at that launch
    B, H, S = 6, 2, 3
    br = Branches(_shape(kind, B, H, L=8, S=S), 340 + kind, 0.3, share=share)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    rng = np.random.default_rng(9 + kind)
    for _ in range(5):
        br.decode(pairs)
    br.fork([0, 0, 2], [3, 4, 5])
    for r in range(6):
        br.spec(S, [int(v) for v in rng.integers(0, S + 1, size=B)], pairs)
        if r == 2:
            br.fork([4], [1])
    for _ in range(3):
        br.decode(pairs)
    br.check(pairs, "fork + speculation")


def _seq_regions(st):
    """(offset, bytes per sequence) of every region of the state, batch outermost."""
    c, L = st.cfg, st.layout
    H, G, P, N, cap = c.heads, c.groups, c.dim_p, c.dim_n, L.ring_cap
    e = 2 if c.in_dtype == bd.SSM_IN_BF16 else 4
    r = [(L.off_ckpt, H * P * N * 4)]
    if c.readcopy == bd.SSM_RC_FP8_ROW:
        r += [(L.off_rc_codes, H * P * N), (L.off_rc_scale, H * P * 4)]
    elif c.readcopy == bd.SSM_RC_FP4_B16:
        r += [(L.off_rc_codes, H * P * N // 2), (L.off_rc_scale, H * P * (N // 16)),
              (L.off_rc_tscale, H * 4)]
    if c.kind == bd.SSM_MAMBA2:
        r += [(L.off_ring[0], H * cap * P * e), (L.off_ring[1], G * cap * N * e),
              (L.off_ring[3], H * cap * 4)]
    else:
        r += [(L.off_ring[1], H * cap * N * e),
              (L.off_ring[2], H * cap * P * e), (L.off_ring[3], H * cap * 4),
              (L.off_ring[4], H * cap * (N if c.kind == bd.SSM_KDA else 1) * 4)]
    r.append((L.off_ptr, H * 16))
    return r


def _rows(st, off, slice_):
    return st.region(off, st.cfg.batch * slice_).view(st.cfg.batch, slice_)


def _same_inputs(d, src, dst):
    d = {k: v.clone() for k, v in d.items()}
    for s, t in zip(src, dst):
        for v in d.values():
            v[t] = v[s]
    return d


@pytest.mark.parametrize("name,rc,share", [
    ("m2_b256", bd.SSM_RC_NONE, 0), ("m2_b256_readcopy", bd.SSM_RC_FP8_ROW, 0),
    ("m2_b256_readcopy", bd.SSM_RC_FP4_B16, 0), ("gdn_b256", bd.SSM_RC_FP8_ROW, 0),
    ("kda_b256", bd.SSM_RC_NONE, 0), ("m2_b256", bd.SSM_RC_NONE, 1),
    ("m2_b256_readcopy", bd.SSM_RC_FP4_B16, 1), ("gdn_b256", bd.SSM_RC_FP8_ROW, 1),
    ("kda_b256", bd.SSM_RC_NONE, 1)])
def test_fork_serving_batch_bit_exact(name, rc, share):
    w = synth.WORKLOADS[name]
    sh = w["shape"]
    br = Branches(sh, w["seed"], w["h0_std"], rc=rc, share=share)
    for _ in range(21):  # a fold, then five buffered entries
        br.decode(None)
    src = list(range(0, 160, 2))           # 80 pairs: more than one launch of the copy
    dst = [s + 1 for s in src]
    before = br.st.mem.clone()
    br.fork(src, dst)
    torch.cuda.synchronize()
    si, di = torch.tensor(src, device=DEV), torch.tensor(dst, device=DEV)
    keep = torch.ones(sh.batch, dtype=torch.bool, device=DEV)
    keep[di] = False
    regions = _seq_regions(br.st)
    ck_off, ck_bytes = br.st.layout.off_ckpt, br.st.layout.off_ring[0] - br.st.layout.off_ckpt
    if share:  # no checkpoint or read-copy byte moves: the copies read the source's slot
        regions = [(o, sl) for (o, sl) in regions if o >= br.st.layout.off_ring[0]]
        assert torch.equal(br.st.mem[ck_off:ck_off + ck_bytes], before[ck_off:ck_off + ck_bytes])
        slot, rcnt = br.slots()
        assert torch.equal(slot[di.cpu()], slot[si.cpu()]) and int(rcnt[src[0]]) == 2
    for (off, sl) in regions:
        now, old = _rows(br.st, off, sl), before[off:off + sh.batch * sl].view(sh.batch, sl)
        assert torch.equal(now[di], now[si]), "region at %d differs after the fork" % off
        assert torch.equal(now[keep], old[keep]), "region at %d changed outside the copies" % off
    del before
    ys = []
    for t in range(13):  # across the next fold
        d = _same_inputs(synth.token_inputs(sh, w["seed"], "branch", 100 + t), src, dst)
        br.decode(None, d)
        ys.append(br.y.clone())
    for t, y in enumerate(ys):
        assert torch.equal(y[di], y[si]), "step %d: a copy's outputs differ from its source" % t
    if share:
        br.check_slots_after_fold()
    bd.ssm_flush(br.st, bd.SSM_FLUSH_ALL)
    nat = torch.empty(sh.batch, sh.heads, sh.dim_p, sh.dim_n, device=DEV)
    bd.ssm_ckpt_export(br.st, nat)
    torch.cuda.synchronize()
    assert torch.equal(nat[di], nat[si])


@pytest.mark.parametrize("name", ["m2_b256", "gdn_b256", "kda_b256"])
def test_restore_serving_batch_sampled(name):
    w = synth.WORKLOADS[name]
    sh = w["shape"]
    br = Branches(sh, w["seed"], w["h0_std"])
    pairs = sample_pairs(sh.batch, sh.heads, 12)
    for _ in range(20):
        br.decode(pairs)
    rng = np.random.default_rng(7)
    br.restore([int(v) for v in rng.integers(-2, 7, size=sh.batch)])
    for _ in range(14):
        br.decode(pairs)
    br.check(pairs, name + " restore")


@pytest.mark.parametrize("kind", [synth.MAMBA2, synth.GDN])
def test_large_batch_past_4gib(kind):
    """Checkpoint regions past 4 GiB (and twice that with shared slots): every offset must be
    formed in 64 bits. Corner and sampled heads against the oracle, across a fork from the last
    sequence into the first and the folds that move the sharers."""
    if kind == synth.MAMBA2:
        shape = synth.Shape(kind, 1024, 128, 128, 64, 128, 16, 1)   # 4 GiB per slot set
    else:
        shape = synth.Shape(kind, 2048, 32, 32, 128, 128, 16, 1)    # 4 GiB per slot set
    B, H = shape.batch, shape.heads
    br = Branches(shape, 500 + kind, 0.3, share=1)
    pairs = sorted(set(sample_pairs(B, H, 10)) | {(1, 0), (B - 2, H - 1)})
    for _ in range(18):  # a fold, then two buffered entries
        br.decode(pairs)
    br.fork([B - 1, 1], [0, B - 2])
    for _ in range(16):  # the next fold moves the sharers to their own slots
        br.decode(pairs)
    br.check(pairs, "large batch")
