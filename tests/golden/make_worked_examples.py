"""Writes worked_examples.json: tiny attention inputs whose exact outputs
follow from closed forms.

Expected values are evaluated here from the closed forms with 50-digit
decimals; this script calls neither the oracle nor the HIP library.  The
pages print no numeric worked example for the forward pass, so each case
cites the passage that defines the quantity it exercises.

Run: python tests/golden/make_worked_examples.py
"""
import decimal
import json
import os

D = decimal.Decimal
CTX = decimal.Context(prec=50)
HD = 64


def sparse(shape, entries):
    return {"shape": shape, "nonzero": [[list(idx), float(val)] for idx, val in entries]}


def main():
    cases = []

    # 1. Two keys with scores 96 and 95 (q = 8 e0, k0 = 96 e0, k1 = 95 e0,
    #    scale 1/8; all exact in bf16).  exp(96) overflows float32, so only a
    #    max-subtracting evaluation is finite.  v0 = e1, v1 = e2, so the output
    #    row holds the two probabilities in columns 1 and 2.
    e1 = CTX.exp(D(-1))
    p0 = CTX.divide(D(1), CTX.add(D(1), e1))
    p1 = CTX.divide(e1, CTX.add(D(1), e1))
    lse = CTX.add(D(96), CTX.ln(CTX.add(D(1), e1)))
    cases.append({
        "name": "two_keys_scores_96_95",
        "cite": "From FlashAttention to FlashAttention 2, section 'Online Softmax' (running "
                "row max m subtracted before exponentiating); FlashAttention-2 from PyTorch to "
                "Triton, definition of L as the logsumexp of the scaled scores",
        "B": 1, "H": 1, "M": 1, "N": 2, "D": HD, "scale": 0.125, "causal": False,
        "q": sparse([1, 1, 1, HD], [((0, 0, 0, 0), 8.0)]),
        "k": sparse([1, 1, 2, HD], [((0, 0, 0, 0), 96.0), ((0, 0, 1, 0), 95.0)]),
        "v": sparse([1, 1, 2, HD], [((0, 0, 0, 1), 1.0), ((0, 0, 1, 2), 1.0)]),
        "o": sparse([1, 1, 1, HD], [((0, 0, 0, 1), str(p0)), ((0, 0, 0, 2), str(p1))]),
        "lse": {"shape": [1, 1, 1], "values": [str(lse)]},
    })

    # 2. Equal scores over two keys whose value rows are 1 + 2^-7 and
    #    1 + 2*2^-7: the mean 1 + 1.5*2^-7 is exactly halfway between two
    #    bf16 neighbours, so a bf16 output shows the rounding mode
    #    (round-to-nearest-even gives 1 + 2*2^-7).  L = log 2.
    a = 1 + 2.0 ** -7
    b = 1 + 2 * 2.0 ** -7
    mean = (a + b) / 2
    cases.append({
        "name": "bf16_rounding_tie",
        "cite": "FlashAttention-2 from PyTorch to Triton, the store of O cast to the output "
                "dtype (the cast rounds; its mode is read as round-to-nearest-even)",
        "B": 1, "H": 1, "M": 3, "N": 2, "D": HD, "scale": 0.125, "causal": False,
        "q": sparse([1, 1, 3, HD], []),
        "k": sparse([1, 1, 2, HD], [((0, 0, 0, 0), 1.0), ((0, 0, 1, 3), -1.0)]),
        "v": {"shape": [1, 1, 2, HD], "fill_rows": [[a] * HD, [b] * HD]},
        "o": {"shape": [1, 1, 3, HD], "fill": mean},
        "o_bf16_rne": 1 + 2 * 2.0 ** -7,
        "lse": {"shape": [1, 1, 3], "values": [str(CTX.ln(D(2)))] * 3},
    })

    # 3. Scores c*j rising along 200 keys (q = e0, k_j = j e0, scale c) with
    #    V_j = (j/256, 1, 0, ...): the maximum moves on every key tile, so every
    #    tile rescales the running state.  l is a geometric series.  (j/256 is
    #    exact in bf16 and keeps |O| < 1, so a bf16 output's rounding stays far
    #    below the tolerance.)
    N = 200
    c = D("0.0625")
    r = CTX.exp(-c)
    l = CTX.divide(CTX.subtract(D(1), CTX.power(r, N)), CTX.subtract(D(1), r))
    L = CTX.add(CTX.multiply(c, D(N - 1)), CTX.ln(l))
    num = D(0)
    for t in range(N):
        num = CTX.add(num, CTX.multiply(D(N - 1 - t), CTX.power(r, t)))
    cases.append({
        "name": "geometric_rising_scores",
        "cite": "FlashAttention-2 from PyTorch to Triton, the online-softmax recurrence "
                "(previous l and O rescaled by exp(m_old - m_new) on every key tile)",
        "B": 1, "H": 1, "M": 1, "N": N, "D": HD, "scale": float(c), "causal": False,
        "q": sparse([1, 1, 1, HD], [((0, 0, 0, 0), 1.0)]),
        "k": sparse([1, 1, N, HD], [((0, 0, j, 0), float(j)) for j in range(1, N)]),
        "v": sparse([1, 1, N, HD], [((0, 0, j, 0), j / 256) for j in range(1, N)]
                    + [((0, 0, j, 1), 1.0) for j in range(N)]),
        "o": sparse([1, 1, 1, HD], [((0, 0, 0, 0), str(CTX.divide(CTX.divide(num, l), D(256)))),
                                    ((0, 0, 0, 1), "1")]),
        "lse": {"shape": [1, 1, 1], "values": [str(L)]},
    })

    # 4. Causal, Q = 0, M = N = 70: row i averages V_0..V_i, L_i = log(i+1);
    #    V_j = (j, 1, 0, ...) so column 0 of row i is i/2.
    M = 70
    cases.append({
        "name": "causal_uniform_prefix",
        "cite": "Writing FlashAttention 2 in Triton, Step 4 (causal mask keeps key <= query, "
                "diagonal included) and its bug catalogue on the comparison direction",
        "B": 1, "H": 1, "M": M, "N": M, "D": HD, "scale": 0.125, "causal": True,
        "q": sparse([1, 1, M, HD], []),
        "k": sparse([1, 1, M, HD], [((0, 0, j, 5), 1.0) for j in range(M)]),
        "v": sparse([1, 1, M, HD], [((0, 0, j, 0), float(j)) for j in range(1, M)]
                    + [((0, 0, j, 1), 1.0) for j in range(M)]),
        "o": sparse([1, 1, M, HD], [((0, 0, i, 0), i / 2) for i in range(1, M)]
                    + [((0, 0, i, 1), 1.0) for i in range(M)]),
        "lse": {"shape": [1, 1, M], "values": [str(CTX.ln(D(i + 1))) for i in range(M)]},
    })

    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_examples.json")
    with open(out, "w") as f:
        json.dump({"about": "closed-form attention cases; see make_worked_examples.py", "cases": cases},
                  f, separators=(",", ":"))
        f.write("\n")
    print("wrote", out)


if __name__ == "__main__":
    main()
