"""The five workload shapes of the round, with their value distributions.

Sizes follow the pages' defaults where they give them: Markov rank r = 256
(pt.news.hada.io, "Arquitetura", Markov head), block length 7 for the offline
evaluation ("Experimentos", setup) and batch 128 for the latency-overhead
measurement ("Análise dos experimentos", overhead paragraph).  The value
distributions and cost tables are synthetic stand-ins: the pages measure on
public math/code/chat suites and live traffic, none of which is used here.

Field meanings
--------------
R, gamma, V, r   requests, block length, vocabulary, Markov rank
w_dtype          "f32" or "bf16" storage of W1 [V, r] and W2 [r, V]
w_sigma          standard deviation of the W1/W2 normal draws
base             "bimodal": N(0,1)*3 with +6 on 2 distinct random tokens per
                 (request, position) row; "peaked": N(0,1)*2 with +8 on 1-3
                 distinct random modes per row (count uniform in {1,2,3})
target           ("const", s): target = base + s*N(0,1) for every request;
                 ("uniform", lo, hi): per-request s ~ U(lo, hi);
                 ("split", s_lo, s_hi): s_lo for requests r < R/2, s_hi after
conf             None (no scheduler, full verify), ("uniform", lo, hi) or
                 ("beta", a, b) per-position conditional confidences
table            None, "linear", "stairs64" or "stairs256_cliff2048"
temperatures     sampling temperatures the workload is run at (0 = greedy)
"""

CONFIGS = {
    1: dict(name="tiny", R=4, gamma=4, V=512, r=16, w_dtype="f32", w_sigma=0.05,
            base="bimodal", target=("const", 0.5), conf=("uniform", 0.5, 1.0),
            table="linear", temperatures=(1.0,)),
    2: dict(name="full_verify_32k", R=32, gamma=7, V=32000, r=256, w_dtype="bf16",
            w_sigma=0.02, base="peaked", target=("const", 0.7), conf=None,
            table=None, temperatures=(1.0,)),
    3: dict(name="scheduled_131k", R=128, gamma=7, V=131072, r=256, w_dtype="bf16",
            w_sigma=0.05, base="bimodal", target=("const", 0.5), conf=("beta", 8.0, 2.0),
            table="stairs64", temperatures=(1.0,)),
    4: dict(name="long_block_chat_mix", R=128, gamma=16, V=131072, r=256, w_dtype="bf16",
            w_sigma=0.05, base="bimodal", target=("uniform", 0.3, 1.5), conf=None,
            table=None, temperatures=(1.0, 0.0)),
    5: dict(name="large_batch_131k", R=512, gamma=16, V=131072, r=256, w_dtype="bf16",
            w_sigma=0.05, base="bimodal", target=("split", 0.3, 1.2), conf=("beta", 6.0, 2.0),
            table="stairs256_cliff2048", temperatures=(1.0,)),
}

# The alternate reading of the 131k scheduled workload: the "peaked" base of the
# 32k workload with its W and target spreads.  Reported as a sensitivity line.
ALTERNATES = {
    "3alt": dict(CONFIGS[3], name="scheduled_131k_peaked", w_sigma=0.02, base="peaked",
                 target=("const", 0.7)),
}


def config(cfg, **overrides):
    """Return a copy of a workload description, with optional field overrides.

    ``cfg`` is an int key of CONFIGS, a key of ALTERNATES, or a dict.
    """
    if isinstance(cfg, dict):
        d = dict(cfg)
    elif cfg in CONFIGS:
        d = dict(CONFIGS[cfg])
    else:
        d = dict(ALTERNATES[cfg])
    d.update(overrides)
    return d
