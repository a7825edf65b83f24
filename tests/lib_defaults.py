"""The library's documented default tile options (include/mk.h, mk_plan_opts),
written out from that documentation for the tests.  These are tuning rules of
the library, not of the pages (which fix no tile size and no split count): the
reference planner in oracle/ takes every option explicitly, and the tests feed
both planners the same values."""


def ceil_div(a, b):
    return -(-a // b)


def documented_defaults(cfg, batch, kv_len, num_cus, **given):
    """Options of a Llama-family plan: 'given' fields as they are, the others by
    the rules mk.h states (ring: 9 pages of 16 KiB at batch 1, 8 above)."""
    H, F, hd, nkv = cfg["hidden"], cfg["ffn"], cfg["head_dim"], cfg["n_kv_heads"]
    o = dict(num_cus=num_cus)
    o["gemv_rows"] = given.get("gemv_rows") or max(4, min(16, 32768 // H))
    o["gateup_outs"] = given.get("gateup_outs") or max(1, o["gemv_rows"] // 2)
    o["down_rows"] = given.get("down_rows") or max(1, min(16, (32768 if batch == 1 else 65536) // F))
    o["lm_rows"] = given.get("lm_rows") or o["gemv_rows"]
    S = given.get("attn_splits")
    if not S:
        n = int(max(kv_len)) + 1
        S = max(1, min(32, ceil_div(n, 64)))
        pairs = batch * nkv
        S = min(S, max(1, ceil_div(2 * num_cus, pairs)))
        cap = 65536
        if pairs * S <= num_cus:
            while S > 1 and pairs * S * 8 > 7 * num_cus:
                S -= 1
            cap = (9 if batch == 1 else 8) * 16384 - 65536
        streams = batch > 1 and hd == 64
        while not streams and ceil_div(n, S) * hd * 2 * 2 > cap:
            S += 1
    o["attn_splits"] = S
    return o


def documented_choices(batch, **given):
    """Planner choices of a Llama-family plan by the rules mk.h states: the
    gcd/lcm events (pairing 0) and longest-first attention at batch > 1
    (attn_order 0 resolves to 1 there, to 0 at batch 1; -1 is plan order),
    in the reference planner's terms (attn_order 1 or 0)."""
    ao = given.get("attn_order", 0)
    return dict(pairing=int(given.get("pairing", 0)), attn_order=(1 if batch > 1 else 0) if ao == 0 else int(ao > 0))
