"""The pages' feed-forward template selector, trained on measured timings.

Digest of "Leveraging Large-Scale Data for Efficient Low-Bit CUTLASS GEMM
Optimization via Neural Networks", Research results items 2-3: every template
is timed on many (M, N, K); a feed-forward network with an input layer, three
hidden layers of width 128 and one output per template, fed the matrix
dimensions and the GPU's multiprocessor count, learns to pick the template;
Adam at learning rate 0.001, batch size 32; judged by top-2 accuracy because
the best and second-best templates run at nearly the same speed.

Readings where the digest is silent or where this build departs from it (also
listed in the design notes):
  - Inputs.  The network sees (M, N, K, CU count) through 18 features computed
    from them: log2 M, log2 N, log2 K, and for each tile size (64, 128 and 256
    square) the log2 of its workgroup count and, for each workgroups-per-CU
    figure that tile size runs at (64: 2, 3, 4; 128: 2, 3; 256: 1), the log2 of
    its number of rounds ceil(tiles / (CU * per-CU)) and the fill of the last
    round.  These make the wave quantisation that decides the fastest tile
    visible to the network: a network fed raw log2 sizes and trained on a
    power-of-two grid picks the large tile at 4568 x 4328, where it runs two
    rounds, the second nearly empty, and is 1.3-1.8x slower than the best.
    Features are standardised with the training set's mean and spread.
  - Outputs and loss.  Output v predicts template v's regret, log(t_v / t_best)
    (times 10), trained with squared error; the selected template has the
    lowest prediction, the runner-up the second lowest.  One-hot labels with
    cross-entropy treat near-ties (templates within 1-2 % of each other, common
    here) as full errors; regression on the regret keeps how close they are.
  - ReLU activations; one network per operand type; 80/20 train/validation
    split by shape with a fixed seed; at most 600 epochs, stopped when the
    validation loss has not improved for 40, keeping the best epoch; five
    initialisations, keeping the one with the lowest validation loss.
  - Training data: the sweep's power-of-two grid plus seeded random shapes
    (the pages' 116,100-sample dataset is not available); scored on a separate
    seeded set of held-out shapes.

  python -m bit_integer_gemm_amd.selector_mlp train grid_s8.jsonl train_s8.jsonl ... --write
  python -m bit_integer_gemm_amd.selector_mlp score heldout_s8.jsonl ...

On one MI355X the CU count is constant; it enters the round features.
"""
from __future__ import annotations

import argparse
import json
import math
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
INC = os.path.join(PKG, "csrc", "selector_mlp.inc")
DTYPES = {"s8": 0, "s4": 1, "b1": 2}
HIDDEN = 128
DEPTH = 3
NCLS = 9
# workgroups per CU at which each tile size runs (LDS and register limits of
# its 2-, 3- and 4-stage variants)
PER_CU = {64: (2, 3, 4), 128: (2, 3), 256: (1,)}
NFEAT = 3 + sum(1 + 2 * len(v) for v in PER_CU.values())   # 18
REGRET_SCALE = 10.0


def features(M, N, K, cu):
    """Raw (unstandardised) feature vector of a shape on a GPU with `cu` CUs."""
    f = [math.log2(M), math.log2(N), math.log2(K)]
    for b, occs in PER_CU.items():
        T = -(-M // b) * -(-N // b)
        f.append(math.log2(T))
        for occ in occs:
            slots = cu * occ
            R = -(-T // slots)
            f.append(math.log2(R))
            f.append(T / (R * slots))
    return np.array(f, dtype=np.float64)


def load(paths):
    """{dtype: {(M, N, K): [t_0 .. t_8]}} from per-shape timing records."""
    out = {}
    for p in paths:
        for line in open(p):
            r = json.loads(line)
            out.setdefault(r["dtype"], {})[(r["M"], r["N"], r["K"])] = r["sec"]
    return out


def regrets(times):
    t = np.asarray(times, np.float64)
    return np.log(t / t.min())


def build_model(torch):
    layers, width = [], NFEAT
    for _ in range(DEPTH):
        layers += [torch.nn.Linear(width, HIDDEN), torch.nn.ReLU()]
        width = HIDDEN
    layers.append(torch.nn.Linear(width, NCLS))
    return torch.nn.Sequential(*layers)


def train(shapes, cu=256, inits=5, log=None):
    """Train networks from `inits` initialisations on one fixed train/validation
    split and keep the one with the lowest validation loss (the held-out shapes
    play no part); returns (weights, mean, spread, info)."""
    best = None
    for init in range(inits):
        net = train_one(shapes, cu=cu, init_seed=init)
        if best is None or net[3]["val_loss"] < best[3]["val_loss"]:
            best = net
    best[3]["inits"] = inits
    if log:
        log(best[3])
    return best


def train_one(shapes, cu=256, max_epochs=600, patience=40, split_seed=0, init_seed=0, log=None):
    """Train one network; returns (weights, mean, spread, info)."""
    import torch
    torch.manual_seed(init_seed)
    keys = sorted(shapes)
    X = np.stack([features(M, N, K, cu) for (M, N, K) in keys])
    Y = np.stack([regrets(shapes[k]) * REGRET_SCALE for k in keys])
    rng = np.random.Generator(np.random.PCG64(split_seed))
    perm = rng.permutation(len(keys))
    nval = max(1, len(keys) // 5)
    val, tr = perm[:nval], perm[nval:]
    mu, sd = X[tr].mean(0), X[tr].std(0) + 1e-9
    Xs = torch.tensor((X - mu) / sd, dtype=torch.float32)
    Yt = torch.tensor(Y, dtype=torch.float32)
    model = build_model(torch)
    opt = torch.optim.Adam(model.parameters(), lr=1e-3, weight_decay=1e-4)
    lossf = torch.nn.MSELoss()
    best = (float("inf"), None, -1)
    g = torch.Generator().manual_seed(init_seed)
    for ep in range(max_epochs):
        model.train()
        order = torch.tensor(tr)[torch.randperm(len(tr), generator=g)]
        for i in range(0, len(order), 32):
            idx = order[i:i + 32]
            opt.zero_grad()
            loss = lossf(model(Xs[idx]), Yt[idx])
            loss.backward()
            opt.step()
        model.eval()
        with torch.no_grad():
            vl = float(lossf(model(Xs[val]), Yt[val]))
        if vl < best[0]:
            best = (vl, {k: v.clone() for k, v in model.state_dict().items()}, ep)
        elif ep - best[2] >= patience:
            break
    model.load_state_dict(best[1])
    ws = [(m.weight.detach().numpy().astype(np.float32), m.bias.detach().numpy().astype(np.float32))
          for m in model if hasattr(m, "weight")]
    info = {"best_epoch": best[2], "val_loss": best[0], "n_train": len(tr), "n_val": len(val),
            "init_seed": init_seed}
    if log:
        log(info)
    return ws, mu.astype(np.float32), sd.astype(np.float32), info


def forward_np(ws, mu, sd, x):
    """Reference forward pass in numpy (fp32): standardise, ReLU layers, scores out."""
    h = ((np.asarray(x, np.float32) - mu) / sd).astype(np.float32)
    for i, (W, b) in enumerate(ws):
        h = W @ h + b
        if i + 1 < len(ws):
            h = np.maximum(h, 0)
    return h


def choose(net, M, N, K, cu=256):
    """(best, second): the two lowest predicted regrets (ties to the lower index)."""
    ws, mu, sd = net
    s = forward_np(ws, mu, sd, features(M, N, K, cu))
    order = sorted(range(NCLS), key=lambda v: (float(s[v]), v))
    return order[0], order[1]


def _hex(a):
    return ",".join(f"0x{x:08x}" for x in np.asarray(a, np.float32).reshape(-1).view(np.uint32))


def write_inc(per_dtype, path=INC):
    """Weights as fp32 bit patterns: per dtype, the feature mean and spread, then
    layers 0..3 (W row-major [out][in], b)."""
    lines = ["// Generated by bit_integer_gemm_amd/selector_mlp.py -- do not edit by hand.",
             f"// Template selector network: {NFEAT} features -> 3 x {HIDDEN} ReLU -> 9 predicted",
             "// regrets (lowest = selected), one network per operand type.",
             f"#define LB_MLP_HIDDEN {HIDDEN}", f"#define LB_MLP_DEPTH {DEPTH}", f"#define LB_MLP_NFEAT {NFEAT}",
             f"static const int kMlpPresent[3] = {{{', '.join('1' if d in per_dtype else '0' for d in DTYPES)}}};"]
    for d, code in DTYPES.items():
        net = per_dtype.get(d)
        mu = net[1] if net else np.zeros(NFEAT, np.float32)
        sd = net[2] if net else np.ones(NFEAT, np.float32)
        lines.append(f"static const uint32_t kMlpMu{code}[{NFEAT}] = {{{_hex(mu)}}};")
        lines.append(f"static const uint32_t kMlpSd{code}[{NFEAT}] = {{{_hex(sd)}}};")
        for li in range(DEPTH + 1):
            fin = NFEAT if li == 0 else HIDDEN
            fout = NCLS if li == DEPTH else HIDDEN
            W, b = net[0][li] if net else (np.zeros((fout, fin), np.float32), np.zeros(fout, np.float32))
            lines.append(f"static const uint32_t kMlpW{code}_{li}[{fout * fin}] = {{{_hex(W)}}};")
            lines.append(f"static const uint32_t kMlpB{code}_{li}[{fout}] = {{{_hex(b)}}};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_inc(path=INC):
    """The generated networks: {code: (weights, mean, spread)}."""
    import re
    text = open(path).read()
    arr = {}
    for m in re.finditer(r"static const uint32_t kMlp(W|B|Mu|Sd)(\d)(?:_(\d))?\[(\d+)\] = \{([^}]*)\};", text):
        kind, code, li, n, body = m.groups()
        vals = np.array([int(v, 16) for v in body.split(",")], np.uint32).view(np.float32)
        arr[(kind, int(code), int(li) if li else -1)] = vals
    present = [x.strip() == "1" for x in re.search(r"kMlpPresent\[3\] = \{([^}]*)\}", text).group(1).split(",")]
    res = {}
    for code in range(3):
        if not present[code] or ("Mu", code, -1) not in arr:
            continue
        ws = []
        for li in range(DEPTH + 1):
            b = arr[("B", code, li)]
            ws.append((arr[("W", code, li)].reshape(len(b), -1), b))
        res[code] = (ws, arr[("Mu", code, -1)], arr[("Sd", code, -1)])
    return res


def score(shapes, pick, eps=0.02, default=7):
    """Held-out scores of a chooser pick(M, N, K) -> (best, second)."""
    def gm(xs):
        return math.exp(sum(math.log(x) for x in xs) / len(xs))
    keys = sorted(shapes)
    sel = [pick(*k) for k in keys]
    ts = [shapes[k] for k in keys]
    fastest = [min(range(NCLS), key=lambda v: (t[v], v)) for t in ts]
    ratio = [t[s[0]] / min(t) for t, s in zip(ts, sel)]
    return {"shapes": len(keys),
            "violations_slower_than_default": sum(1 for t, s in zip(ts, sel) if t[s[0]] > (1 + eps) * t[default]),
            "top2_accuracy": sum(1 for s, f in zip(sel, fastest) if f in s) / len(keys),
            "top1_within_eps": sum(1 for r in ratio if r <= 1 + eps) / len(keys),
            "selected_over_fastest": {"geomean": gm(ratio), "worst": max(ratio)},
            "speedup_vs_default_geomean": gm([t[default] / t[s[0]] for t, s in zip(ts, sel)])}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("train")
    t.add_argument("files", nargs="+")
    t.add_argument("--write", action="store_true")
    t.add_argument("--json")
    s = sub.add_parser("score")
    s.add_argument("files", nargs="+")
    s.add_argument("--json")
    a = ap.parse_args(argv)
    if a.cmd == "train":
        data = load(a.files)
        per, report = {}, {}
        for d in DTYPES:
            if d not in data:
                continue
            ws, mu, sd, info = train(data[d], log=lambda i, d=d: print(d, i, flush=True))
            per[d] = (ws, mu, sd)
            report[d] = info
        if a.write:
            write_inc(per)
            print(f"wrote {INC}")
        if a.json:
            json.dump(report, open(a.json, "w"), indent=1)
    else:
        nets = read_inc()
        rep = {}
        for d, shapes in load(a.files).items():
            net = nets[DTYPES[d]]
            rep[d] = score(shapes, lambda M, N, K: choose(net, M, N, K))
        print(json.dumps(rep, indent=1))
        if a.json:
            json.dump(rep, open(a.json, "w"), indent=1)


if __name__ == "__main__":
    main()
