"""Pure-Python transcription of the oracle, for tiny inputs only.

TEST INFRASTRUCTURE ONLY.  It exists to cross-check the C oracle's indexing and strides on small
random cases (two independent transcriptions of the same sequential recurrence); it is not a pin
of the arithmetic itself -- the pins are the printed values, closed forms and brute-force forms
in the oracle pin tests.

Same reading as the C oracle: Delta = softplus(raw + bias) when requested, Abar = exp(Delta*A),
Bbar*x = Delta*B*u, h_t = Abar*h_{t-1} + Bbar*x_t from h = 0, y_t = sum_n C*h_t (+ D*u) (* silu z).
"""
import math


def _softplus(x):
    return max(x, 0.0) + math.log1p(math.exp(-abs(x)))


def scan_loops(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False):
    """Nested lists / numpy arrays in, nested lists (out, last_state) out."""
    batch, dim, L = len(u), len(u[0]), len(u[0][0])
    N = len(A[0])
    out = [[[0.0] * L for _ in range(dim)] for _ in range(batch)]
    last = [[[0.0] * N for _ in range(dim)] for _ in range(batch)]
    for b in range(batch):
        for d in range(dim):
            h = [0.0] * N
            for t in range(L):
                dt = float(delta[b][d][t]) + (float(delta_bias[d]) if delta_bias is not None else 0.0)
                if delta_softplus:
                    dt = _softplus(dt)
                x = float(u[b][d][t])
                y = 0.0
                for n in range(N):
                    h[n] = math.exp(dt * float(A[d][n])) * h[n] + dt * float(B[b][n][t]) * x
                    y += float(C[b][n][t]) * h[n]
                if D is not None:
                    y += float(D[d]) * x
                if z is not None:
                    zz = float(z[b][d][t])
                    y *= zz / (1.0 + math.exp(-zz))
                out[b][d][t] = y
            last[b][d] = list(h)
    return out, last
