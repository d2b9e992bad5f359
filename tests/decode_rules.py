"""The decode launch rules that the header states, restated for the tests
(test infrastructure): which calls split grouped-head work evenly."""


def even_split(S, Hq, Hkv, P, parts):
    """Whether pa_decode splits the batch's work evenly over the resident
    workgroups: a supported group size (1, 2, 4 or 8 query heads per KV head),
    more than one partition of P tokens, at most 1024 sequences, split
    positions within 32 bits, and for one or two heads per KV head more than
    2,048 partitions in all (8 per compute unit of 256)."""
    G = Hq // Hkv
    if G not in (1, 2, 4, 8) or parts < 2 or S > 1024:
        return False
    if G <= 2 and S * Hkv * parts <= 2048:
        return False
    units = S * Hkv * parts * (P // 16)
    return units + S * Hkv * parts + 8 + 9 * (P // 16) < (1 << 31)
