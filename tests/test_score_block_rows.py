"""The merged score block of the FP8-cache kernel computes the next tile's
row addresses, and loads the page ids of the unit after next, in inline asm
(gen_score_blocks.row_ops).  This emulates that instruction sequence lane by
lane on the host and checks it against the rules the C++ path applies
(stage_row, fetch_page): token t of the lane's load slot, the zero row past
the row length or for a page outside the pool, the page-range flag only for
tokens inside the row, the page-table entry of the token (entry 0 past the
row).  No GPU needed."""
import os
import random
import re
import sys

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "decode_context_parallelism_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_score_blocks as G  # noqa: E402

M32 = (1 << 32) - 1
M64 = (1 << 64) - 1


def tok_slot(t):
    return 16 * (t >> 4) + 8 * ((t >> 2) & 1) + 4 * ((t >> 3) & 1) + (t & 3)


def load_slot(wave, lane):
    return (16 * (wave & 1) + (lane & 15)) ^ (8 * ((lane >> 4) & 1))


def page_addresses(wave, s2, lmax2, shift, pt2):
    out = []
    for lane in range(64):
        t = s2 * 64 + 32 * (wave >> 1) + tok_slot(load_slot(wave, lane))
        out.append(pt2 + 4 * ((t >> shift) if t < lmax2 else 0))
    return out


def reference(wave, s, lmax, pages, shift, num_pages, pool, zero):
    rows, bad = [], False
    for lane in range(64):
        t = s * 64 + 32 * (wave >> 1) + tok_slot(load_slot(wave, lane))
        in_seq = t < lmax
        ok = 0 <= pages[lane] < num_pages
        bad = bad or (in_seq and not ok)
        if in_seq and ok:
            r = (pages[lane] << shift) + (t & ((1 << shift) - 1))
            rows.append(pool + r * 576 + 16 * (lane >> 4))
        else:
            rows.append(zero + 16 * (lane >> 4))
    return rows, bad


def s32(x):
    x &= M32
    return x - (1 << 32) if x >> 31 else x


def emulate(ops, sregs):
    """Run the row ops on 64 lanes.  sregs: the asm's scalar operands by name;
    %[page] is per lane (a list)."""
    v = [dict() for _ in range(64)]          # per-lane VGPRs
    masks = {}                               # SGPR pairs / vcc as 64-bit lane masks
    loads = []                               # per-lane addresses of each global load

    def val(lane, x):
        x = x.strip()
        m = re.fullmatch(r"%\[(\w+)\]", x)
        if m:
            sv = sregs[m.group(1)]
            return sv[lane] if isinstance(sv, list) else sv
        if x.startswith("v["):
            lo = int(x[2:].split(":")[0])
            return v[lane][lo] | (v[lane][lo + 1] << 32)
        if x.startswith("v"):
            return v[lane][int(x[1:])]
        return int(x, 0)

    def put(lane, d, x):
        if d.startswith("v["):
            lo = int(d[2:].split(":")[0])
            v[lane][lo], v[lane][lo + 1] = x & M32, (x >> 32) & M32
        else:
            v[lane][int(d[1:])] = x & M32

    for op in ops:
        name, rest = op.split(None, 1)
        a = [x.strip() for x in rest.split(",")]
        if name in ("s_andn2_b64", "s_and_b64"):
            x, y = masks[a[1].strip("%[]")], masks[a[2].strip("%[]")]
            masks[a[0].strip("%[]")] = (x & ~y) & M64 if name == "s_andn2_b64" else x & y
            continue
        if name == "global_load_dword":
            loads.append([val(lane, a[1]) for lane in range(64)])
            continue
        if name.startswith("v_cmp"):
            m = 0
            for lane in range(64):
                x, y = val(lane, a[1]), val(lane, a[2])
                c = s32(x) > s32(y) if name == "v_cmp_gt_i32" else (x & M32) > (y & M32)
                m |= int(c) << lane
            masks[a[0].strip("%[]")] = m
            continue
        for lane in range(64):
            if name == "v_mbcnt_lo_u32_b32":      # bits of -1 below the lane, low half
                put(lane, a[0], min(lane, 32))
            elif name == "v_mbcnt_hi_u32_b32":    # plus those of the high half
                put(lane, a[0], val(lane, a[2]) + max(lane - 32, 0))
            elif name == "v_lshrrev_b32":
                put(lane, a[0], (val(lane, a[2]) & M32) >> (val(lane, a[1]) & 31))
            elif name == "v_and_b32":
                put(lane, a[0], val(lane, a[1]) & val(lane, a[2]))
            elif name == "v_xor_b32":
                put(lane, a[0], val(lane, a[1]) ^ val(lane, a[2]))
            elif name == "v_mul_u32_u24":
                put(lane, a[0], (val(lane, a[1]) & 0xFFFFFF) * (val(lane, a[2]) & 0xFFFFFF))
            elif name == "v_add_u32":
                put(lane, a[0], val(lane, a[1]) + val(lane, a[2]))
            elif name == "v_lshl_add_u32":
                put(lane, a[0], ((val(lane, a[1]) << val(lane, a[2])) & M32) + val(lane, a[3]))
            elif name == "v_mov_b32":
                put(lane, a[0], val(lane, a[1]))
            elif name == "v_lshl_add_u64":
                put(lane, a[0], ((val(lane, a[1]) << val(lane, a[2])) + val(lane, a[3])) & M64)
            elif name == "v_mad_u64_u32":
                put(lane, a[0], ((val(lane, a[2]) & M32) * (val(lane, a[3]) & M32) + val(lane, a[4])) & M64)
            elif name == "v_cndmask_b32":
                sel = (masks[a[3]] >> lane) & 1
                put(lane, a[0], val(lane, a[2]) if sel else val(lane, a[1]))
            else:
                raise AssertionError(f"unemulated instruction {name}")
    rows = [v[lane][230] | (v[lane][231] << 32) for lane in range(64)]
    return rows, masks["badm"] != 0, loads


def _case(rng, wave, shift, s, lmax, num_pages, bad_pages, s2=None, lmax2=None):
    pages = [rng.randrange(num_pages) for _ in range(64)]
    for lane in rng.sample(range(64), bad_pages):
        pages[lane] = rng.choice([-1, -7, num_pages, num_pages + 123, 0x7FFFFFFF])
    pool, zero = 0x7F3A_0000_0000 + 256 * rng.randrange(1 << 20), 0x7F00_1234_5600
    ts = s * 64 + 32 * (wave >> 1) + 16 * (wave & 1)
    np_ = min(num_pages, 0x7FFFFFFF)
    s2 = s + 1 if s2 is None else s2
    lmax2 = lmax + 64 if lmax2 is None else lmax2
    pt2 = 0x7E00_0000_0000 + 4 * rng.randrange(1 << 20)
    sregs = {"page": [p & M32 for p in pages], "ts": ts, "lmax": lmax, "mask": (1 << shift) - 1,
             "shift": shift, "np": np_, "pool": pool, "zero": zero,
             "ts2": s2 * 64 + 32 * (wave >> 1) + 16 * (wave & 1), "lmax2": lmax2, "pt2": pt2}
    got_rows, got_bad, loads = emulate(G.row_ops(), sregs)
    want_rows, want_bad = reference(wave, s, lmax, pages, shift, num_pages, pool, zero)
    assert got_rows == want_rows
    assert got_bad == want_bad
    assert loads == [page_addresses(wave, s2, lmax2, shift, pt2)]


def test_row_ops_match_stage_row_rules():
    rng = random.Random(7)
    for _ in range(300):
        wave = rng.randrange(4)
        shift = rng.choice([0, 1, 3, 4, 6, 9])
        s = rng.randrange(4096)
        lmax = s * 64 + rng.randrange(-8, 72)          # row ends before, inside or after the stage
        num_pages = rng.choice([1, 17, 5000, 1 << 20])
        s2 = rng.choice([s + 1, rng.randrange(4096)])      # the unit after next: any row position
        lmax2 = s2 * 64 + rng.randrange(-8, 72)
        _case(rng, wave, shift, s, lmax, num_pages, rng.choice([0, 0, 1, 5]), s2, lmax2)


def test_row_ops_flag_only_visible_bad_pages():
    rng = random.Random(11)
    # every page outside the pool, but the row ends before the stage: zero rows, no flag
    _case(rng, 1, 3, 10, 10 * 64, 50, 64)
    # the same pages with the whole stage visible: zero rows and the flag
    _case(rng, 2, 3, 10, 11 * 64, 50, 64)
