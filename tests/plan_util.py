"""The producer/consumer kernel's plan restated in Python (the tests compare
the library's lowram_decode_plan with it, and use it to say which cases run
several tiles or several heads per workgroup)."""


def pipe_plan(heads, n_tiles, n_cu=256):
    """The library's plan for the producer/consumer kernel, restated to document
    what each case exercises: groups of t tiles (t >= 2 where a head has 2)
    dealt round-robin to W = min(n_cu, groups) workgroups, t giving the fewest
    ceil(groups / W) * t, the largest on ties.  Returns (W, t, groups per head,
    the most tiles one workgroup runs, whether some workgroup runs several heads)."""
    best = None
    for t in range(min(2, n_tiles), n_tiles + 1):
        groups = heads * -(-n_tiles // t)
        w = min(n_cu, groups)
        cost = -(-groups // w) * t
        if best is None or cost <= best[0]:
            best = (cost, t)
    t = best[1]
    n_grp = -(-n_tiles // t)
    groups = heads * n_grp
    w = min(n_cu, groups)
    size = [min(t, n_tiles - (g % n_grp) * t) for g in range(groups)]
    load = [sum(size[g] for g in range(i, groups, w)) for i in range(w)]
    several = any(len({g // n_grp for g in range(i, groups, w)}) > 1 for i in range(w))
    return w, t, n_grp, max(load), several
