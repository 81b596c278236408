"""A tiny fp64 recurrent "trunk" and drafter for end-to-end checks of the cycle.

Test infrastructure.  It stands in for the target model so that speculative decoding can
be compared with ordinary decoding token by token and state byte by state byte.

  state  S [H][n][n]   per-head matrix updated by a delta-rule-style step driven by the
                       consumed token: S_h <- g S_h Q_h + beta (v - S_h kappa) kappa^T
                       (Q_h orthogonal, g < 1, so the state keeps moving)
  hidden h = tanh(P vec(S) - a E[tok])              (the row the LM head reads)
  head   W = E + noise (tied embeddings; with -a E[tok] in h, repeats are discouraged)
  KV     one appended row per consumed token: R E[tok]
  drafter: the same map with a perturbed P and its own running copy of the state
"""
import numpy as np


class ToyTrunk:
    def __init__(self, seed: int, V: int = 24, d: int = 16, H: int = 2, n: int = 4,
                 kv_dim: int = 6, draft_noise: float = 0.12):
        rng = np.random.default_rng(seed)
        self.V, self.d, self.H, self.n, self.kv_dim = V, d, H, n, kv_dim
        self.E = rng.standard_normal((V, d))
        self.Ak = rng.standard_normal((H, n, d)) / np.sqrt(d)
        self.Av = rng.standard_normal((H, n, d)) / np.sqrt(d)
        self.c = rng.standard_normal((H, d)) / np.sqrt(d)
        self.P = rng.standard_normal((d, H * n * n)) * 0.8
        self.Pd = self.P + rng.standard_normal(self.P.shape) * draft_noise
        self.R = rng.standard_normal((kv_dim, d))
        self.Q = np.stack([np.linalg.qr(rng.standard_normal((n, n)))[0] for _ in range(H)])
        self.W = (self.E + 0.5 * rng.standard_normal((V, d))) * 1.5      # shared LM head

    def zero_state(self) -> np.ndarray:
        return np.zeros((self.H, self.n, self.n))

    def step(self, S: np.ndarray, tok: int) -> np.ndarray:
        e = self.E[tok]
        S = S.copy()
        for h in range(self.H):
            kappa = self.Ak[h] @ e
            kappa /= max(np.linalg.norm(kappa), 1e-12)
            v = self.Av[h] @ e
            beta = 1.0 / (1.0 + np.exp(-(self.c[h] @ e)))
            S[h] = 0.97 * S[h] @ self.Q[h] + beta * np.outer(v - S[h] @ kappa, kappa)
        return S

    def hidden(self, S: np.ndarray, tok: int, drafter: bool = False) -> np.ndarray:
        P = self.Pd if drafter else self.P
        return np.tanh(P @ S.reshape(-1) - 1.2 * self.E[tok])

    def kv_row(self, tok: int) -> np.ndarray:
        return (self.R @ self.E[tok]).astype(np.float64)

    @staticmethod
    def state_bytes(S: np.ndarray) -> np.ndarray:
        return np.frombuffer(np.ascontiguousarray(S, dtype=np.float64).tobytes(), dtype=np.uint8).copy()


class ToyTrunkConv(ToyTrunk):
    """The toy trunk with a short causal convolution in front of each recurrent update
    (as the gated-delta layers of the pages' model have): the state is the matrices S plus
    the last C inputs, so rolling back needs the conv rows too.  State = one float64
    vector [vec(S), conv rows], padded to a whole number of 16-byte words."""

    def __init__(self, seed: int, C: int = 3, **kw):
        super().__init__(seed, **kw)
        rng = np.random.default_rng(seed + 1000)
        self.C = C
        self.cw = rng.standard_normal(C) / C + np.eye(1, C, C - 1)[0]      # last tap dominant
        self.ns = self.H * self.n * self.n
        self.size = self.ns + C * self.d
        self.size += self.size % 2

    def zero_state(self) -> np.ndarray:
        return np.zeros(self.size)

    def _split(self, st):
        S = st[:self.ns].reshape(self.H, self.n, self.n)
        conv = st[self.ns:self.ns + self.C * self.d].reshape(self.C, self.d)
        return S, conv

    def step(self, st: np.ndarray, tok: int) -> np.ndarray:
        S, conv = self._split(st)
        conv = np.concatenate([conv[1:], self.E[tok][None]], axis=0)
        x = self.cw @ conv                                                 # short conv over the inputs
        S = S.copy()
        for h in range(self.H):
            kappa = self.Ak[h] @ x
            kappa /= max(np.linalg.norm(kappa), 1e-12)
            v = self.Av[h] @ x
            beta = 1.0 / (1.0 + np.exp(-(self.c[h] @ x)))
            S[h] = 0.97 * S[h] @ self.Q[h] + beta * np.outer(v - S[h] @ kappa, kappa)
        out = np.zeros(self.size)
        out[:self.ns] = S.reshape(-1)
        out[self.ns:self.ns + self.C * self.d] = conv.reshape(-1)
        return out

    def hidden(self, st: np.ndarray, tok: int, drafter: bool = False) -> np.ndarray:
        S, conv = self._split(st)
        P = self.Pd if drafter else self.P
        return np.tanh(P @ S.reshape(-1) - 1.2 * (self.cw @ conv))

    @staticmethod
    def state_bytes(st: np.ndarray) -> np.ndarray:
        return np.frombuffer(np.ascontiguousarray(st, dtype=np.float64).tobytes(), dtype=np.uint8).copy()

    @staticmethod
    def from_bytes(b: np.ndarray) -> np.ndarray:
        return np.frombuffer(np.ascontiguousarray(b).tobytes(), dtype=np.float64).copy()
