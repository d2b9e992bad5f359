"""The decode launch rules that the header states, restated for the tests
(test infrastructure): which calls split grouped-head work evenly."""


def even_split(S, Hq, Hkv, P, parts):
    """Whether pa_decode splits the batch's work evenly over the resident
    workgroups: groups of 4 or 8 query heads, more than one partition of P
    tokens, at most 1024 sequences, split positions within 32 bits."""
    G = Hq // Hkv
    if G not in (4, 8) or parts < 2 or S > 1024:
        return False
    units = S * Hkv * parts * (P // 16)
    return units + S * Hkv * parts + 8 + 9 * (P // 16) < (1 << 31)
