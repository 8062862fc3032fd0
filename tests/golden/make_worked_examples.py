"""Writes the two hand-worked fixtures in this folder.

The expected values are closed forms (sums of powers of e) derived by hand
from SP-KV section 2.1, Eq. (1)-(4); this script only evaluates them.  It
calls neither the oracle nor the HIP library.
"""
import os
import json, math
e = math.e
T, nq, nkv, hd, w = 5, 4, 2, 4, 2
z = [[1,0],[0,1],[0,0],[1,0],[0,0]]
k0_g0 = [1, 9, 0, 2, 0]
k0_g1 = [5, -1, 7, 1, 3]
c_g1  = [0.25, 0.5, 1.5, 0.0, -0.5]
K = [[[k0_g0[s], 1.0, -1.0, 2.0], [k0_g1[s], 0.0, 0.0, c_g1[s]]] for s in range(T)]
V = [[[s+1, 10*(s+1), -(s+1), (s+1)**2], [100+s, s, 2*s, 0.5*s]] for s in range(T)]
q = [[2,0,0,0],[0,0,0,0],[2,0,0,0],[0,0,0,4]]
Q = [q for _ in range(T)]
def comb(ps, rows):
    S = sum(ps)
    return [sum(p*r[d] for p, r in zip(ps, rows))/S for d in range(hd)], math.log(S)
exp = {}
# t = 4: kv0 visible {0,3,4} scores (dim0 carrier) 1,2,0 ; kv1 visible {1,3,4}
V0 = [V[s][0] for s in range(T)]; V1 = [V[s][1] for s in range(T)]
exp["4"] = [comb([e, e**2, 1], [V0[0], V0[3], V0[4]]),
            comb([1, 1, 1], [V0[0], V0[3], V0[4]]),
            comb([e**-1, e, e**3], [V1[1], V1[3], V1[4]]),
            comb([e, 1, e**-1], [V1[1], V1[3], V1[4]])]
# t = 0: only s = 0
exp["0"] = [comb([1], [V0[0]]), comb([1], [V0[0]]), comb([1], [V1[0]]), comb([1], [V1[0]])]
exp["0"] = [(o, l) for (o, _), l in zip(exp["0"], [1.0, 0.0, 5.0, 0.5])]
# t = 2: kv0 visible {0,1,2}; kv1 visible {1,2}
exp["2"] = [comb([e, e**9, 1], [V0[0], V0[1], V0[2]]),
            comb([1, 1, 1], [V0[0], V0[1], V0[2]]),
            comb([e**-1, e**7], [V1[1], V1[2]]),
            comb([e, e**3], [V1[1], V1[2]])]
fx = {
 "source": "Self-Pruned Key-Value Attention (arXiv 2605.14037), section 2.1, Eq. (3)-(4): windowed-plus-gated softmax attention",
 "what": "hand-worked example; expected values are closed forms in e, evaluated to double precision",
 "derivation": [
   "scale = 1/sqrt(hd) = 1/2; query heads 0 and 2 are [2,0,0,0] so the score of key s is its first component; head 1 is zero (uniform weights); head 3 is [0,0,0,4] so the score is 2*k_s[3]",
   "heads 0,1 read key head 0 and heads 2,3 read key head 1 (contiguous groups of n_q/n_kv = 2)",
   "w = 2: the window of row t is {t-1, t}; key head 0 keeps s in {0,3}, key head 1 keeps s = 1",
   "t = 4: key head 0 sees {0,3,4} (scores 1,2,0 for head 0), key head 1 sees {1,3,4} (scores -1,1,3 for head 2; 1,0,-1 for head 3)",
   "t = 0: every head sees only s = 0, so out = v_0 and lse = the score of s = 0",
   "t = 2: key head 0 sees {0,1,2} (scores 1,9,0), key head 1 sees {1,2} (scores -1,7 for head 2; 1,3 for head 3)",
   "out = sum_s exp(x_s) v_s / sum_s exp(x_s), lse = log sum_s exp(x_s)"
 ],
 "T": T, "n_q": nq, "n_kv": nkv, "head_dim": hd, "window": w, "scale": 0.5,
 "z": z, "K": K, "V": V, "Q": Q,
 "rows": [4, 0, 2],
 "expected_out": {t: [o for o, _ in exp[t]] for t in exp},
 "expected_lse": {t: [l for _, l in exp[t]] for t in exp},
}
json.dump(fx, open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "attention_worked_example.json"), "w"), indent=1)

# gate example: d_model 2, d_hidden 3, n_kv 2
gx = {
 "source": "Self-Pruned Key-Value Attention (arXiv 2605.14037), section 2.1, Eq. (1)-(2): u = sigmoid(f(h)), z = [u >= tau]; f a 2-layer MLP (ReLU, biases)",
 "what": "hand-worked example",
 "derivation": [
   "h = [1, -2]",
   "W1 h + b1 = [1*1 + 1*(-2) + 0.5, 2*1 + (-1)*(-2) + 0, 0*1 + 0.5*(-2) + 1] = [-0.5, 4, 0]",
   "ReLU -> a = [0, 4, 0]",
   "logit_0 = 3*0 + 0.25*4 + (-7)*0 + (-1) = 0 -> u_0 = 0.5 -> kept at tau = 0.5 (>=)",
   "logit_1 = 1*0 + (-0.5)*4 + 2*0 + 3 = 1 -> u_1 = 1/(1+e^-1)",
   "second row h = [0, 0]: a = ReLU(b1) = [0.5, 0, 1]; logit_0 = 1.5 - 7 - 1 = -6.5; logit_1 = 0.5 + 2 + 3 = 5.5"
 ],
 "H": [[1.0, -2.0], [0.0, 0.0]],
 "W1": [[1.0, 1.0], [2.0, -1.0], [0.0, 0.5]],
 "b1": [0.5, 0.0, 1.0],
 "W2": [[3.0, 0.25, -7.0], [1.0, -0.5, 2.0]],
 "b2": [-1.0, 3.0],
 "tau": 0.5,
 "expected_logit": [[0.0, 1.0], [-6.5, 5.5]],
 "expected_u": [[0.5, 1/(1+math.exp(-1))], [1/(1+math.exp(6.5)), 1/(1+math.exp(-5.5))]],
 "expected_z": [[1, 1], [0, 1]],
}
json.dump(gx, open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "gate_worked_example.json"), "w"), indent=1)
