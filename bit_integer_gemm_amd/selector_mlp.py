"""The feed-forward template classifier of the pages, trained on measured sweeps.

Digest of "Leveraging Large-Scale Data for Efficient Low-Bit CUTLASS GEMM
Optimization via Neural Networks", Research results item 3: a feed-forward
network with an input layer, three hidden layers of width 128 and an output
layer over the nine templates; inputs are the matrix dimensions (M, N, K) and
the GPU's multiprocessor count; trained with cross-entropy and Adam at learning
rate 0.001 with batch size 32; judged by top-2 accuracy because the best and
second-best templates run at nearly the same speed.

Readings where the digest is silent (also listed in the design notes): ReLU
activations; inputs scaled as (log2 M, log2 N, log2 K) divided by 16 and the CU
count divided by 256; one network per operand type (the templates differ per
type); the label of a shape is its fastest variant in the training sweep; 80/20
train/validation split by shape with a fixed seed; a fixed number of epochs
with the validation loss tracked and the best epoch kept.

  python -m bit_integer_gemm_amd.selector_mlp train sweep_s8_run1.jsonl sweep_s4_run1.jsonl \\
         sweep_b1_run1.jsonl --write        # writes csrc/selector_mlp.inc
  python -m bit_integer_gemm_amd.selector_mlp score sweep_s8_run2.jsonl ...   # vs independent run

On one MI355X the CU count is constant, so that input carries no information
here; it is kept so that the network has the pages' inputs.
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


def features(M, N, K, cu):
    return np.array([math.log2(M) / 16.0, math.log2(N) / 16.0, math.log2(K) / 16.0, cu / 256.0],
                    dtype=np.float32)


def load_sweep(paths):
    """{dtype: {(M, N, K): [t_0 .. t_8]}} from sweep JSON lines."""
    out = {}
    for p in paths:
        for line in open(p):
            r = json.loads(line)
            if r["variant"] == "auto":   # the library's own choice, not one of the nine
                continue
            out.setdefault(r["dtype"], {}).setdefault((r["M"], r["N"], r["K"]), [None] * 9)[r["variant"]] = r["sec"]
    return {d: {k: v for k, v in s.items() if None not in v} for d, s in out.items()}


def build_model(torch):
    layers, width = [], 4
    for _ in range(DEPTH):
        layers += [torch.nn.Linear(width, HIDDEN), torch.nn.ReLU()]
        width = HIDDEN
    layers.append(torch.nn.Linear(width, NCLS))
    return torch.nn.Sequential(*layers)


def train_one(shapes, cu=256, epochs=600, seed=0, log=None):
    import torch
    torch.manual_seed(seed)
    keys = sorted(shapes)
    X = np.stack([features(M, N, K, cu) for (M, N, K) in keys])
    y = np.array([int(np.argmin(shapes[k])) for k in keys])
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(len(keys))
    nval = max(1, len(keys) // 5)
    val, tr = perm[:nval], perm[nval:]
    model = build_model(torch)
    opt = torch.optim.Adam(model.parameters(), lr=1e-3)
    lossf = torch.nn.CrossEntropyLoss()
    Xt, yt = torch.from_numpy(X), torch.from_numpy(y)
    best = (float("inf"), None, -1)
    g = torch.Generator().manual_seed(seed)
    for ep in range(epochs):
        model.train()
        order = torch.from_numpy(tr)[torch.randperm(len(tr), generator=g)]
        for i in range(0, len(order), 32):
            idx = order[i:i + 32]
            opt.zero_grad()
            loss = lossf(model(Xt[idx]), yt[idx])
            loss.backward()
            opt.step()
        model.eval()
        with torch.no_grad():
            vl = float(lossf(model(Xt[val]), yt[val]))
        if vl < best[0]:
            best = (vl, {k: v.detach().clone() for k, v in model.state_dict().items()}, ep)
    model.load_state_dict(best[1])
    model.eval()
    with torch.no_grad():
        logits = model(Xt).numpy()
    acc = lambda idx: topk_acc(logits[idx], [shapes[keys[i]] for i in idx])  # noqa: E731
    info = {"train": acc(tr), "val": acc(val), "best_epoch": best[2], "val_loss": best[0],
            "n_train": len(tr), "n_val": len(val)}
    if log:
        log(info)
    return model, info


def topk_acc(logits, times):
    """(top-1, top-2) accuracy: is the measured fastest variant among the k highest logits?"""
    t1 = t2 = 0
    for lg, ts in zip(logits, times):
        best = int(np.argmin(ts))
        order = np.argsort(-lg)
        t1 += int(order[0] == best)
        t2 += int(best in order[:2])
    n = max(1, len(times))
    return t1 / n, t2 / n


def weights_of(model):
    ws = []
    for m in model:
        if hasattr(m, "weight"):
            ws.append((m.weight.detach().numpy().astype(np.float32), m.bias.detach().numpy().astype(np.float32)))
    return ws


def forward_np(ws, x):
    """Reference forward pass in numpy (fp32): ReLU between layers, logits out."""
    h = np.asarray(x, np.float32)
    for i, (W, b) in enumerate(ws):
        h = W @ h + b
        if i + 1 < len(ws):
            h = np.maximum(h, 0)
    return h


def write_inc(per_dtype, path=INC):
    """Weights as C arrays: for each dtype, layers 0..3 (W row-major [out][in], b)."""
    lines = ["// Generated by bit_integer_gemm_amd/selector_mlp.py -- do not edit by hand.",
             "// Feed-forward template classifier: 4 inputs -> 3 x 128 ReLU -> 9 logits, per dtype.",
             f"#define LB_MLP_HIDDEN {HIDDEN}", f"#define LB_MLP_DEPTH {DEPTH}",
             f"static const int kMlpPresent[3] = {{{', '.join('1' if d in per_dtype else '0' for d in DTYPES)}}};"]
    for d, code in DTYPES.items():
        ws = per_dtype.get(d)
        for li in range(DEPTH + 1):
            fin = 4 if li == 0 else HIDDEN
            fout = NCLS if li == DEPTH else HIDDEN
            if ws is None:
                W = np.zeros((fout, fin), np.float32)
                b = np.zeros(fout, np.float32)
            else:
                W, b = ws[li]
            # fp32 bit patterns: exact, and half the text of decimal or hex-float literals
            wl = ",".join(f"0x{x:08x}" for x in W.astype(np.float32).reshape(-1).view(np.uint32))
            bl = ",".join(f"0x{x:08x}" for x in b.astype(np.float32).reshape(-1).view(np.uint32))
            lines.append(f"static const uint32_t kMlpW{code}_{li}[{fout * fin}] = {{{wl}}};")
            lines.append(f"static const uint32_t kMlpB{code}_{li}[{fout}] = {{{bl}}};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_inc(path=INC):
    """Parse the generated weights back (for tests): {code: [(W, b)] * 4}."""
    import re
    text = open(path).read()
    out = {}
    for m in re.finditer(r"static const uint32_t kMlp([WB])(\d)_(\d)\[(\d+)\] = \{([^}]*)\};", text):
        kind, code, li, n, body = m.groups()
        vals = np.array([int(v, 16) for v in body.split(",")], np.uint32).view(np.float32)
        out.setdefault(int(code), {}).setdefault(int(li), {})[kind] = vals
    res = {}
    for code, layers in out.items():
        ws = []
        for li in sorted(layers):
            b = layers[li]["B"]
            W = layers[li]["W"].reshape(len(b), -1)
            ws.append((W, b))
        res[code] = ws
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("train")
    t.add_argument("files", nargs="+")
    t.add_argument("--epochs", type=int, default=600)
    t.add_argument("--write", action="store_true")
    t.add_argument("--json")
    s = sub.add_parser("score")
    s.add_argument("files", nargs="+")
    s.add_argument("--json")
    a = ap.parse_args(argv)
    if a.cmd == "train":
        data = load_sweep(a.files)
        per, report = {}, {}
        for d in DTYPES:
            if d not in data:
                continue
            model, info = train_one(data[d], epochs=a.epochs, log=lambda i, d=d: print(d, i, flush=True))
            per[d] = weights_of(model)
            report[d] = info
        if a.write:
            write_inc(per)
            print(f"wrote {INC}")
        if a.json:
            json.dump(report, open(a.json, "w"), indent=1)
    else:
        data = load_sweep(a.files)
        weights = read_inc()
        rep = {}
        for d, shapes in data.items():
            ws = weights[DTYPES[d]]
            keys = sorted(shapes)
            logits = np.stack([forward_np(ws, features(M, N, K, 256)) for (M, N, K) in keys])
            t1, t2 = topk_acc(logits, [shapes[k] for k in keys])
            sel = [int(np.argmax(lg)) for lg in logits]
            sp = [shapes[k][7] / shapes[k][v] for k, v in zip(keys, sel)]
            viol = sum(1 for k, v in zip(keys, sel) if shapes[k][v] > 1.02 * shapes[k][7])
            gm = math.exp(sum(math.log(x) for x in sp) / len(sp))
            rep[d] = {"shapes": len(keys), "top1": t1, "top2": t2, "speedup_vs_default_geomean": gm,
                      "violations_slower_than_default": viol}
        print(json.dumps(rep, indent=1))
        if a.json:
            json.dump(rep, open(a.json, "w"), indent=1)


if __name__ == "__main__":
    main()
