"""Host-only checks of the C ABI: the libraries load, export every entry point
that include/*.h declares (include/skinny.h: libskinny; include/skinny_ceiling.h:
the benchmark's measurement references, libskinny_ceiling), every declaration
cites the passage of the pages that defines it, and the host logic (argument
checks, the launch-shape chooser, error reasons) behaves as documented.  No
compute call is made here: these tests run without a GPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PRODUCT_HEADER = "skinny.h"
CEILING_HEADER = "skinny_ceiling.h"

# The pages' sections a declaration may cite (page title tail, then section).
PAGES = {
    "unpooler": ["module description", "Unpooler.run", "Unpooler.unsupported", "Unpooler",
                 "compile_unpooler", "launch_unsupported"],
    "pooler_gather": ["module description", "Pooler", "PoolerGemmShape", "PoolerLayer",
                      "compile_norm_quant", "compile_gather", "compile_pooler_gemm",
                      "cvt_e2m1x8_f32", "cvt_f32_to_e4m3", "nvfp4_compute_output_scale"],
    "oproj.batt": ["module description", "AttentionBoundary", "OProjection"],
}
# Declarations that are not steps of the method say so instead of citing.
NOT_A_STEP = ("Not a step of the method", "For callers that cannot allocate")


def _header_text(header):
    with open(os.path.join(ROOT, "include", header)) as f:
        return f.read()


def _declarations(header):
    """[(name, comment)] for every function the header declares; the comment
    is the last comment between the previous declaration and this one (a
    declaration right after another shares that one's comment)."""
    text = _header_text(header)
    out, prev_end, prev_comment = [], 0, ""
    for m in re.finditer(r"^(?:int|const char \*|void)\s*(skinny_\w+)\s*\(", text, flags=re.M):
        between = text[prev_end:m.start()]
        comments = re.findall(r"/\*.*?\*/", between, flags=re.S)
        comment = comments[-1] if comments else prev_comment
        out.append((m.group(1), comment))
        prev_end = text.index(";", m.end()) + 1
        prev_comment = comment
    return out


def _declared_symbols(header=None):
    headers = [header] if header else [h for h in os.listdir(os.path.join(ROOT, "include"))
                                       if h.endswith(".h")]
    names = set()
    for h in headers:
        text = re.sub(r"/\*.*?\*/", "", _header_text(h), flags=re.S)
        names |= set(re.findall(r"\b(skinny_\w+)\s*\(", text))
    return sorted(names)


def _cites_a_passage(comment):
    body = re.sub(r"^\s*/?\*+/?", "", comment, flags=re.M).replace("*/", "")
    flat = " ".join(body.split())
    if any(tag in flat for tag in NOT_A_STEP):
        return True
    for page, sections in PAGES.items():
        for m in re.finditer(re.escape(page) + r" page[,:]? ", flat):
            tail = flat[m.end():m.end() + 200]
            if any(tail.startswith(sec) or f" {sec}" in tail[:120] for sec in sections):
                return True
    return False


@pytest.fixture(scope="module")
def sk():
    import moe_decode_skinny_amd as sk

    return sk


def test_headers_are_the_two_libraries():
    assert sorted(h for h in os.listdir(os.path.join(ROOT, "include")) if h.endswith(".h")) == \
        [PRODUCT_HEADER, CEILING_HEADER]


def test_header_declares_the_entry_points():
    names = _declared_symbols(PRODUCT_HEADER)
    for n in ["skinny_init", "skinny_gemm_bf16", "skinny_rmsnorm_nvfp4", "skinny_choose",
              "skinny_last_error"]:
        assert n in names
    assert not [n for n in names if n.startswith("skinny_ceiling")]


@pytest.mark.parametrize("header", [PRODUCT_HEADER, CEILING_HEADER])
def test_every_declaration_cites_its_passage(header):
    """Each declared call's comment names a page and one of its sections, or
    says that it is not a step of the method."""
    decls = _declarations(header)
    assert sorted(n for n, _ in decls) == _declared_symbols(header)
    bad = [n for n, c in decls if not _cites_a_passage(c)]
    assert not bad, bad


def test_citation_check_rejects_uncited_comments():
    assert not _cites_a_passage("/* The same GEMM at an explicit launch. */")
    assert not _cites_a_passage("/* the unpooler page */")
    assert _cites_a_passage("/* (unpooler page,\n * launch_unsupported) */")


def test_library_exports_every_declared_symbol(sk):
    lib = ctypes.CDLL(sk.LIB_PATH)
    missing = [n for n in _declared_symbols(PRODUCT_HEADER) if not hasattr(lib, n)]
    assert not missing, missing
    # the measurement references live only in their own library
    assert not hasattr(lib, "skinny_ceiling_stream") and not hasattr(lib, "skinny_ceiling_empty")
    assert not hasattr(lib, "skinny_ceiling_stream_store")


def test_ceiling_library_exports_its_symbols():
    from moe_decode_skinny_amd import ceiling

    lib = ctypes.CDLL(ceiling.LIB_PATH)
    missing = [n for n in _declared_symbols(CEILING_HEADER) if not hasattr(lib, n)]
    assert not missing, missing
    for n in _declared_symbols(CEILING_HEADER):
        assert hasattr(ceiling, n), n


def test_binding_has_the_same_names(sk):
    for n in _declared_symbols(PRODUCT_HEADER):
        assert hasattr(sk, n), n


def test_version(sk):
    assert sk.skinny_version() >= 100


@pytest.mark.parametrize("M,N,K", [(m, 1024, 4096) for m in (1, 2, 4, 8, 16)]
                         + [(m, 8192, 1024) for m in (1, 8, 16)]
                         + [(m, 512, 8192) for m in (1, 8, 16)]
                         + [(m, 4096, 8192) for m in (1, 8, 16)]
                         + [(3, 48, 40), (16, 16, 8), (1, 16, 8), (5, 208, 1000)])
@pytest.mark.parametrize("splits", [0, 1, 2, 4, 8, 16])
def test_chooser_gives_valid_launches(sk, M, N, K, splits):
    reason = sk.skinny_gemm_unsupported(M, N, K, splits)
    if reason is not None:
        # only an explicit split count too small for a long K may be refused
        assert splits in (1, 2) and "too long" in reason, reason
        return
    launch = sk.skinny_choose(M, N, K, splits)
    assert sk.skinny_launch_unsupported(M, N, K, launch) is None
    assert sk.skinny_gemm_unsupported(M, N, K, splits) is None
    if splits:
        assert launch.splits == splits
    # waves = F * ceil(K / (splits * kw)): kw = 32 * chunks and F = rows / 16
    # tiles (MFMA), or kw = 512 * chunks (DOT2) or 128 * chunks (MFMA 4x4)
    # and F = 1
    mfma = launch.path == sk.SKINNY_PATH_MFMA
    kw = {sk.SKINNY_PATH_MFMA: 32, sk.SKINNY_PATH_DOT2: 512,
          sk.SKINNY_PATH_MFMA_4X4: 128}[launch.path] * launch.chunks
    F = launch.rows // 16 if mfma else 1
    assert launch.waves == F * -(-K // (launch.splits * kw))
    # pure: the same arguments give the same launch
    assert sk.skinny_choose(M, N, K, splits) == launch


@pytest.mark.parametrize(
    "M,N,K,splits,needle",
    [(0, 1024, 4096, 0, "M=0"), (17, 1024, 4096, 0, "M=17"), (1, 1000, 4096, 0, "N=1000"),
     (1, 0, 4096, 0, "N=0"), (1, 1024, 4095, 0, "K=4095"), (1, 1024, 0, 0, "K=0"),
     (1, 1024, 4096, 3, "splits=3"), (1, 1024, 4096, 32, "splits=32"),
     (1, 16, (1 << 25) + 8, 0, "at most"), (1, (1 << 24) + 16, 8, 0, "at most"),
     (4, 16, 524288 + 8, 0, "K too long"), (8, 16, 262144 + 8, 0, "K too long"),
     (16, 16, 131072 + 8, 0, "K too long")],
)
def test_unsupported_reasons(sk, M, N, K, splits, needle):
    reason = sk.skinny_gemm_unsupported(M, N, K, splits)
    assert reason is not None and needle in reason
    with pytest.raises(ValueError, match=re.escape(needle)):
        sk.skinny_choose(M, N, K, splits)


def test_launch_unsupported_reasons(sk):
    L = sk.Launch
    assert "splits" in sk.skinny_launch_unsupported(1, 1024, 4096, L(1, 3, 8, 4, 1, 16))
    assert "chunks" in sk.skinny_launch_unsupported(1, 1024, 4096, L(1, 4, 8, 3, 1, 16))
    assert "waves" in sk.skinny_launch_unsupported(1, 1024, 4096, L(1, 4, 4, 4, 1, 16))
    assert "rows" in sk.skinny_launch_unsupported(1, 1024, 4096, L(1, 4, 8, 4, 1, 8))
    assert "waves" in sk.skinny_launch_unsupported(1, 1024, 4096, L(1, 4, 8, 4, 1, 32))
    assert sk.skinny_launch_unsupported(1, 1024, 4096, L(1, 4, 16, 4, 1, 32)) is None
    assert "workspace" in sk.skinny_launch_unsupported(16, 16384, 4096, L(1, 16, 8, 1, 1, 16))
    assert sk.skinny_launch_unsupported(16, 1024, 4096, L(1, 1, 16, 8, 1, 16)) is None
    assert "DOT2" in sk.skinny_launch_unsupported(16, 1024, 4096, L(0, 1, 8, 1, 1, 16))
    assert "multiple" in sk.skinny_launch_unsupported(1, 1040, 4096, L(0, 1, 8, 1, 1, 32))
    assert sk.skinny_launch_unsupported(1, 1024, 4096, L(0, 1, 8, 1, 1, 4)) is None
    assert sk.skinny_launch_unsupported(16, 1024, 4096, L(1, 4, 8, 4, 2, 16)) is None


@pytest.mark.parametrize("N,K", [(1024, 4096), (8192, 1024), (512, 8192), (4096, 8192), (48, 1000)])
@pytest.mark.parametrize("M", range(1, 17))
def test_chooser_walk(sk, M, N, K):
    """skinny_choose_walk describes what skinny_gemm_bf16 runs: the plain
    kernel at skinny_choose's launch, or a valid one-item ring launch with the
    same arithmetic (the staged MFMA ring standing for the MFMA launch)."""
    launch = sk.skinny_choose(M, N, K, 0)
    walk = sk.skinny_choose_walk(M, N, K, 0)
    if walk.segment == 0:
        assert walk.gemm == launch and walk.workgroups == 0
    else:
        g = walk.gemm
        if g.path == sk.SKINNY_PATH_MFMA_LDS:
            g = g._replace(path=sk.SKINNY_PATH_MFMA)
        assert g == launch
        assert sk.skinny_ring_launch_unsupported(M, N, K, 1, walk) is None
    assert sk.skinny_choose_walk(M, N, K, 0) == walk


def test_chooser_walks_the_measured_shapes(sk):
    """The shapes whose single calls measured faster as a persistent walk."""
    for M, N, K in [(2, 8192, 1024), (8, 8192, 1024), (16, 8192, 1024), (3, 4096, 8192),
                    (8, 4096, 8192), (16, 4096, 8192)]:
        assert sk.skinny_choose_walk(M, N, K, 0).segment > 0, (M, N, K)
    for M, N, K in [(1, 1024, 4096), (2, 1024, 4096), (4, 1024, 4096), (16, 1024, 4096),
                    (1, 8192, 1024), (4, 8192, 1024)]:
        assert sk.skinny_choose_walk(M, N, K, 0).segment == 0, (M, N, K)
    with pytest.raises(ValueError, match="M=17"):
        sk.skinny_choose_walk(17, 1024, 4096, 0)


def test_off_table_staged_walks(sk):
    """Off the table, 9..16 tokens with K <= 4096 on N >= 2048 run the MFMA
    launch of 16 rows x 16 chunks as the staged walk: one segment a
    workgroup, at most 256 workgroups; fewer tokens, narrow N, long K, an
    explicit split count and the 16-block rule's shapes do not."""
    for M, N, K, seg, wgs in [(16, 8192, 2048, 2, 256), (12, 4096, 1024, 1, 256),
                              (9, 2048, 1000, 1, 128), (16, 16384, 1024, 4, 256),
                              (16, 8192, 3072, 2, 256), (16, 8192, 4096, 2, 256),
                              (12, 4096, 4096, 1, 256)]:
        w = sk.skinny_choose_walk(M, N, K, 0)
        l = sk.skinny_choose(M, N, K, 0)
        assert (w.gemm.path, w.segment, w.workgroups) == (sk.SKINNY_PATH_MFMA_LDS, seg, wgs)
        assert (l.path, l.splits, l.chunks, l.rows, l.waves) == (1, 1, 16, 16, -(-K // 512))
    for M, N, K, splits in [(8, 8192, 2048, 0), (16, 1024, 2048, 0), (16, 8192, 8192, 0),
                            (16, 8192, 2048, 2), (16, 2048, 4096, 0)]:
        w = sk.skinny_choose_walk(M, N, K, splits)
        assert w.segment == 0 or w.gemm.path != sk.SKINNY_PATH_MFMA_LDS, (M, N, K, splits)


def test_off_table_16_block_walks(sk):
    """The rule's 16-block launches on 512 or more output blocks run as walks
    of one segment per workgroup, the segment as long as keeps 256 or more
    workgroups; fewer blocks run the plain kernel."""
    P3 = sk.SKINNY_PATH_MFMA_4X4
    for M, N, K, seg, wgs in [(16, 2048, 8192, 2, 256), (12, 8192, 8192, 8, 256),
                              (9, 3072, 6144, 2, 384), (16, 2064, 4096, 2, 258)]:
        w = sk.skinny_choose_walk(M, N, K, 0)
        assert (w.gemm.path, w.segment, w.workgroups) == (P3, seg, wgs), (M, N, K, w)
        assert tuple(w.gemm) == tuple(sk.skinny_choose(M, N, K, 0))
        assert w.gemm.accs == 1 and w.gemm.rows == 4
    for M, N, K in [(16, 1040, 6000), (16, 1024, 8192), (12, 2032, 4096), (9, 2048, 4096)]:
        w = sk.skinny_choose_walk(M, N, K, 0)
        assert w.gemm.path == P3 and w.segment == 0, (M, N, K, w)


def test_off_table_dot2_walks(sk):
    """3-8 tokens (and 2 at K = 8192) on wide off-table shards run the DOT2
    walk: 2 chunks a wave, K / 1024 waves, 4 rows up to K = 4096 and 2
    above, 256 workgroups of one or two segments of 2, 4 or 8 blocks;
    skinny_choose returns the walk's launch. No walk when the blocks do not
    split that evenly, at 1 token, at 2 tokens below K = 8192, at 3-4 tokens
    unless K is a multiple of 4096, or outside 4096..8192."""
    P0 = sk.SKINNY_PATH_DOT2
    for M, N, K, seg, rows in [(3, 2048, 4096, 2, 4), (8, 4096, 4096, 4, 4),
                               (4, 8192, 4096, 8, 4), (6, 16384, 4096, 8, 4),
                               (5, 2048, 8192, 4, 2), (8, 8192, 8192, 8, 2),
                               (5, 2048, 6144, 4, 2), (8, 4096, 5120, 8, 2),
                               (2, 2048, 8192, 4, 2), (2, 8192, 8192, 8, 2)]:
        w = sk.skinny_choose_walk(M, N, K, 0)
        assert (w.gemm.path, w.segment, w.workgroups) == (P0, seg, 256), (M, N, K, w)
        assert (w.gemm.waves, w.gemm.chunks, w.gemm.rows) == (K // 1024, 2, rows), (M, N, K, w)
        assert tuple(w.gemm) == tuple(sk.skinny_choose(M, N, K, 0))
    for M, N, K in [(2, 4096, 4096), (1, 8192, 8192), (8, 3072, 4096), (8, 6144, 8192),
                    (4, 2048, 6144), (3, 4096, 5120), (8, 2048, 3072), (8, 2048, 9216),
                    (8, 1536, 4096)]:
        w = sk.skinny_choose_walk(M, N, K, 0)
        assert w.segment == 0, (M, N, K, w)
    # an explicit split count keeps the plain rule
    assert sk.skinny_choose_walk(8, 4096, 4096, 2).segment == 0


def test_rule_takes_the_16_block_path_for_many_tokens_on_long_k(sk):
    """The chooser outside the table for 9..16 tokens and 4096 <= K <= 8192:
    the 16-block MFMA with one split, 4 chunks, and the rows (4 or 8) and
    token groups (1 or 2) that give the most workgroups in 128..256, ties
    to fewer rows + tokens a workgroup; with none in that range, 4 rows and
    one group when N / 4 >= 256; DOT2 or the 16x16 MFMA otherwise (fewer
    tokens, narrow N, short or very long K)."""
    P3 = sk.SKINNY_PATH_MFMA_4X4
    for M, N, K, rows, H in [(9, 1024, 4096, 8, 2), (12, 2048, 4096, 8, 1),
                             (16, 1040, 6000, 4, 1), (16, 2048, 8192, 4, 1),
                             (16, 512, 4096, 4, 2), (12, 768, 8192, 8, 2),
                             (9, 1536, 4096, 8, 1), (12, 1008, 4096, 8, 2)]:
        l = sk.skinny_choose(M, N, K, 0)
        assert (l.path, l.splits, l.chunks, l.rows, l.accs) == (P3, 1, 4, rows, H), (M, N, K, l)
        assert l.waves == -(-K // 512)
    for M, N, K, splits in [(8, 2048, 4096, 0), (12, 240, 4096, 0), (12, 2048, 2048, 0),
                            (12, 2048, 8200, 0), (8, 1024, 4096, 2)]:
        assert sk.skinny_choose(M, N, K, splits).path != P3, (M, N, K, splits)


def test_rule_sums_requested_splits_inside_the_16_block_kernel(sk):
    """An explicit split count S > 1 for 9..16 tokens and 4096 <= K <= 8192:
    the 16-block launch of 8 rows, 4 chunks, two token groups up to
    N = 1024 (one above), whose splits the last workgroup of each output
    block sums, when that is at most 2048 workgroups; else the DOT2 or MFMA
    split launch."""
    P3 = sk.SKINNY_PATH_MFMA_4X4
    for M, N, K, S, H in [(16, 512, 8192, 4, 2), (9, 1024, 4096, 2, 2), (12, 2048, 4096, 2, 1),
                          (16, 4096, 8192, 4, 1), (16, 8192, 8192, 2, 1)]:
        l = sk.skinny_choose(M, N, K, S)
        assert tuple(l) == (P3, S, -(-K // (S * 512)), 4, H, 8), (M, N, K, S, l)
        assert N // 8 * H * S <= 2048
    for M, N, K, S in [(16, 8192, 8192, 4), (16, 8192, 1024, 2), (8, 512, 8192, 4)]:
        assert sk.skinny_choose(M, N, K, S).path != P3, (M, N, K, S)


def test_mfma_4x4_token_groups(sk):
    """Token groups (accs = H) of the 16-block path: group h takes tokens
    4Qh .. 4Qh + 4Q - 1 with Q the token sets of ceil(M / H) (1, 2 or 4),
    and every group needs a token (ceil(M / 4Q) == H). The ring and the
    chooser's walks keep all tokens in one workgroup, and a grid over 2^32
    work-items is refused."""
    L, P = sk.Launch, sk.SKINNY_PATH_MFMA_4X4
    ok = {(M, H) for M in range(1, 17) for H in (1, 2, 4)
          if sk.skinny_launch_unsupported(M, 1024, 4096, L(P, 1, 8, 4, H, 4)) is None}
    # H = 1: every M; H = 2: M = 5..16 (4 or 8 tokens a group); H = 4: M = 13..16
    assert ok == ({(M, 1) for M in range(1, 17)} | {(M, 2) for M in range(5, 17)}
                  | {(M, 4) for M in range(13, 17)})
    for M, H in [(4, 2), (12, 4), (9, 4), (16, 3), (16, 0), (16, 8)]:
        why = sk.skinny_launch_unsupported(M, 1024, 4096, L(P, 1, 8, 4, H, 4))
        assert why is not None and f"accs={H}" in why, (M, H, why)
    # token groups with splits: valid, the splits' workspace as without them
    assert sk.skinny_launch_unsupported(16, 512, 8192, L(P, 2, 8, 4, 2, 4)) is None
    assert sk.skinny_launch_unsupported(13, 512, 8192, L(P, 4, 4, 4, 4, 4)) is None
    ring = sk.RingLaunch(L(P, 1, 8, 4, 2, 4), 1, 256, 0)
    assert "all M tokens" in sk.skinny_ring_launch_unsupported(16, 1024, 4096, 1, ring)
    # 2^22 blocks of 4 rows x 4 token groups x 16 waves: 2^34 work-items
    why = sk.skinny_launch_unsupported(16, 1 << 24, 8192, L(P, 1, 16, 4, 4, 4))
    assert why is not None and "2^32 work-items" in why, why
    assert "2^32 work-items" in sk.skinny_launch_unsupported(16, 1 << 24, 8192,
                                                             L(P, 1, 16, 4, 1, 4))


def test_mfma_4x4_launch_reasons(sk):
    """The 16-block MFMA path: rows 4 or 8, accs = token groups 1, 2 or 4
    (each with a token), chunks 4 or 8 (whole 512-K load groups),
    waves = ceil(K / (S * 128 chunks)) <= 16, and only the register-budgeted
    variants."""
    L, P = sk.Launch, sk.SKINNY_PATH_MFMA_4X4
    assert sk.skinny_launch_unsupported(16, 1024, 4096, L(P, 1, 8, 4, 1, 4)) is None
    assert sk.skinny_launch_unsupported(16, 1024, 4096, L(P, 2, 4, 4, 1, 8)) is None
    assert sk.skinny_launch_unsupported(1, 512, 8192, L(P, 1, 16, 4, 1, 4)) is None
    assert "rows=2" in sk.skinny_launch_unsupported(16, 1024, 4096, L(P, 1, 8, 4, 1, 2))
    assert "rows=16" in sk.skinny_launch_unsupported(16, 1024, 4096, L(P, 1, 8, 4, 1, 16))
    assert "accs=3" in sk.skinny_launch_unsupported(16, 1024, 4096, L(P, 1, 8, 4, 3, 4))
    assert "needs 8 waves" in sk.skinny_launch_unsupported(16, 1024, 4096, L(P, 1, 4, 4, 1, 4))
    assert "MFMA 4x4: 1..16" in sk.skinny_launch_unsupported(16, 1024, 16384,
                                                            L(P, 1, 32, 4, 1, 4))
    for chunks in (1, 2, 16):
        assert "needs 4 or 8" in sk.skinny_launch_unsupported(
            16, 1024, 4096, L(P, 1, 4096 // (128 * chunks), chunks, 1, 4))
    # 8 rows x 8 chunks x 16 tokens needs 224 registers a lane: not built
    assert "no MFMA 4x4 kernel" in sk.skinny_launch_unsupported(16, 1024, 4096,
                                                                L(P, 1, 4, 8, 1, 8))
    # the same at 1024 threads (112 registers): 4 rows x 4 chunks x 16 tokens is 96
    assert sk.skinny_launch_unsupported(16, 512, 8192, L(P, 1, 16, 4, 1, 4)) is None
    assert "no MFMA 4x4 kernel" in sk.skinny_launch_unsupported(16, 512, 8192,
                                                                L(P, 1, 16, 4, 1, 8))


def test_compute_calls_without_device_fail_cleanly(sk):
    # Pointer checks come before any device access: null pointers are EINVAL.
    lib = ctypes.CDLL(sk.LIB_PATH)
    lib.skinny_gemm_bf16.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    assert lib.skinny_gemm_bf16(None, None, None, 1, 1024, 4096, 0, None) == sk.SKINNY_EINVAL
    assert lib.skinny_gemm_bf16(16, 32, 48, 17, 1024, 4096, 0, None) == sk.SKINNY_EINVAL
    # misaligned
    assert lib.skinny_gemm_bf16(18, 4096, 1 << 20, 1, 1024, 4096, 0, None) == sk.SKINNY_EINVAL
    assert "aligned" in sk.skinny_last_error()
    # y overlapping W
    assert lib.skinny_gemm_bf16(0x10000, 0x100000, 0x100010, 1, 16, 64, 0, None) == sk.SKINNY_EINVAL
    assert "overlap" in sk.skinny_last_error()
    lib.skinny_rmsnorm_nvfp4.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                         ctypes.c_float] + [ctypes.c_void_p] * 3 + \
                                        [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.skinny_rmsnorm_nvfp4(0x1000, 0x2000, 1.0, 1e-6, 0x3000, 0x4000, 0x5000, 8, 4100,
                                    None) == sk.SKINNY_EINVAL
    assert "P=4100" in sk.skinny_last_error()


@pytest.mark.parametrize("M,N,K", [(m, 1024, 4096) for m in (1, 2, 4, 8, 16)]
                         + [(m, 8192, 1024) for m in (1, 8, 16)]
                         + [(m, 512, 8192) for m in (1, 8, 16)]
                         + [(m, 4096, 8192) for m in (1, 8, 16)]
                         + [(3, 48, 1000), (16, 16, 8), (1, 16, 8), (16, 1024, 6000)])
@pytest.mark.parametrize("count", [1, 7, 64])
def test_ring_chooser_gives_valid_launches(sk, M, N, K, count):
    r = sk.skinny_ring_choose(M, N, K, count)
    g = r.gemm
    assert g.splits == 1
    if g.path == sk.SKINNY_PATH_DOT2:
        assert g.accs == 1 and g.waves == -(-K // (512 * g.chunks)) <= 16
        if g.waves <= 8:  # the single-call DOT2 kernel has up to 8 waves
            assert sk.skinny_launch_unsupported(M, N, K, g) is None
    elif g.path == sk.SKINNY_PATH_MFMA_4X4:
        assert g.accs == 1 and g.rows in (4, 8) and g.waves == -(-K // (128 * g.chunks)) <= 16
        # the ring's launch is also a valid single-call launch (same arithmetic)
        assert sk.skinny_launch_unsupported(M, N, K, g) is None
    else:
        assert g.waves == g.rows // 16 * -(-K // (32 * g.chunks)) <= 16
    groups = N // g.rows
    assert N % g.rows == 0 and groups % r.segment == 0
    assert 1 <= r.workgroups <= count * groups // r.segment
    assert sk.skinny_ring_launch_unsupported(M, N, K, count, r) is None
    assert sk.skinny_ring_choose(M, N, K, count) == r


def test_ring_rule_off_the_table(sk):
    """The ring chooser off the table: 5..16 tokens take the staged MFMA ring
    in 32-block segments over 240 workgroups (K <= 4096) or the 16-block ring
    over 256; 1..4 tokens the DOT2 ring with 4 rows, 2 chunks, 4-block
    segments over 1024 workgroups; all in XCD-local order; few items shorten
    the segment first, then the workgroup count."""
    X = sk.SKINNY_RING_XCD_LOCAL
    cases = [((16, 2048, 4096, 60), (2, 16, 16, 32, 240)), ((8, 8192, 2048, 60), (2, 16, 16, 32, 240)),
             ((16, 2048, 8192, 60), (3, 4, 4, 32, 256)), ((2, 4096, 2048, 60), (0, 2, 4, 4, 1024)),
             ((4, 2048, 8192, 60), (0, 2, 4, 4, 1024)), ((16, 2048, 4096, 3), (2, 16, 16, 1, 240)),
             ((1, 1024, 8192, 3), (0, 2, 4, 1, 768))]
    for (M, N, K, count), (path, chunks, rows, seg, wgs) in cases:
        r = sk.skinny_ring_choose(M, N, K, count)
        got = (r.gemm.path, r.gemm.chunks, r.gemm.rows, r.segment, r.workgroups)
        assert got == (path, chunks, rows, seg, wgs) and r.order == X, (M, N, K, count, r)
        assert sk.skinny_ring_launch_unsupported(M, N, K, count, r) is None


def test_ring_unsupported_shapes_and_reasons(sk):
    with pytest.raises(ValueError, match="count=0"):
        sk.skinny_ring_choose(1, 1024, 4096, 0)
    with pytest.raises(ValueError, match="count=65"):
        sk.skinny_ring_choose(1, 1024, 4096, 65)
    with pytest.raises(ValueError, match="M=17"):
        sk.skinny_ring_choose(17, 1024, 4096, 1)
    # 16 tokens at K = 16384: 32 waves of one chunk, more than a workgroup
    with pytest.raises(ValueError, match="no ring launch"):
        sk.skinny_ring_choose(16, 4096, 16384, 2)


def _ring_lib(sk):
    lib = ctypes.CDLL(sk.LIB_PATH)
    lib.skinny_gemm_bf16_ring_launch.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4 + [
        ctypes.POINTER(sk._CRingLaunch), ctypes.c_void_p]
    lib.skinny_gemm_bf16_ring.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4 + [
        ctypes.c_void_p]
    return lib


def _ptrs(*vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def test_ring_launch_reasons_without_device(sk):
    lib = _ring_lib(sk)
    M, N, K = 1, 1024, 4096
    x, w, y = _ptrs(0x100000), _ptrs(0x1000000), _ptrs(0x4000000)

    def call(gemm, seg=1, wg=None, count=1):
        if wg is None:
            wg = N // gemm[5] // seg
        c = sk.RingLaunch(sk.Launch(*gemm), seg, wg)._c()
        return lib.skinny_gemm_bf16_ring_launch(x, w, y, count, M, N, K, ctypes.byref(c), None)

    assert call((1, 1, 16, 4, 1, 16)) == sk.SKINNY_EUNSUPPORTED  # MFMA: K needs 32 waves
    assert "needs 32 waves" in sk.skinny_last_error()
    assert call((1, 1, 16, 8, 4, 16)) == sk.SKINNY_EUNSUPPORTED
    assert "MFMA ring kernel" in sk.skinny_last_error()
    assert call((1, 1, 16, 8, 1, 48)) == sk.SKINNY_EUNSUPPORTED
    assert "rows=48" in sk.skinny_last_error()
    assert call((2, 1, 16, 8, 1, 16)) == sk.SKINNY_EUNSUPPORTED  # staged: LDS too small
    assert "167936 bytes of LDS" in sk.skinny_last_error()
    assert call((2, 1, 16, 1, 1, 16)) == sk.SKINNY_EUNSUPPORTED
    assert "MFMA_LDS ring kernel" in sk.skinny_last_error()
    assert call((4, 1, 16, 8, 1, 16)) == sk.SKINNY_EUNSUPPORTED
    assert "unknown path" in sk.skinny_last_error()
    assert call((3, 1, 16, 8, 1, 16)) == sk.SKINNY_EUNSUPPORTED  # MFMA 4x4: rows 4 or 8
    assert "MFMA 4x4 rows=16" in sk.skinny_last_error()
    assert call((3, 1, 8, 8, 1, 4)) == sk.SKINNY_EUNSUPPORTED  # K=4096 at 8 chunks: 4 waves
    assert "needs 4 waves" in sk.skinny_last_error()
    assert call((3, 1, 4, 8, 2, 4)) == sk.SKINNY_EUNSUPPORTED
    assert "accs=1" in sk.skinny_last_error()
    # 8 rows x 8 chunks x 16 tokens: 288 registers a lane, more than any form has
    c = sk.RingLaunch(sk.Launch(3, 1, 4, 8, 1, 8), 1, 128)._c()
    assert lib.skinny_gemm_bf16_ring_launch(x, w, y, 1, 16, N, K, ctypes.byref(c), None) == \
        sk.SKINNY_EUNSUPPORTED
    assert "MFMA 4x4 ring kernel" in sk.skinny_last_error()
    assert call((3, 1, 8, 4, 1, 4)) in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)
    assert call((2, 1, 8, 16, 1, 16)) in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)
    assert call((0, 2, 1, 4, 1, 2)) == sk.SKINNY_EUNSUPPORTED
    assert "splits=1" in sk.skinny_last_error()
    c = sk.RingLaunch(sk.Launch(0, 1, 2, 4, 1, 2), 1, 512, 2)._c()
    assert lib.skinny_gemm_bf16_ring_launch(x, w, y, 1, M, N, K, ctypes.byref(c), None) == \
        sk.SKINNY_EUNSUPPORTED
    assert "order=2" in sk.skinny_last_error()
    c = sk.RingLaunch(sk.Launch(0, 1, 2, 4, 1, 2), 1, 512, sk.SKINNY_RING_XCD_LOCAL)._c()
    assert lib.skinny_gemm_bf16_ring_launch(x, w, y, 1, M, N, K, ctypes.byref(c), None) in (
        sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)
    assert call((0, 1, 3, 4, 1, 2)) == sk.SKINNY_EUNSUPPORTED
    assert "waves" in sk.skinny_last_error()
    assert call((0, 1, 2, 4, 1, 2), wg=513) == sk.SKINNY_EUNSUPPORTED
    assert "workgroups=513" in sk.skinny_last_error()
    assert call((0, 1, 2, 4, 1, 2), seg=3, wg=1) == sk.SKINNY_EUNSUPPORTED
    assert "segment=3" in sk.skinny_last_error()
    assert call((0, 1, 2, 4, 1, 2), seg=4, wg=129) == sk.SKINNY_EUNSUPPORTED
    assert "workgroups=129" in sk.skinny_last_error()
    assert call((0, 1, 2, 4, 1, 16)) == sk.SKINNY_EUNSUPPORTED
    assert "ring kernel" in sk.skinny_last_error()
    assert call((0, 1, 2, 4, 1, 2), count=65) == sk.SKINNY_EINVAL
    # valid launches pass every check and stop at the missing device
    assert call((1, 1, 16, 8, 1, 16)) in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)
    assert call((0, 1, 2, 4, 1, 2)) in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)
    assert call((0, 1, 2, 4, 1, 2), seg=512, wg=1) in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)


def test_ring_rejects_aliased_items_without_device(sk):
    lib = _ring_lib(sk)
    M, N, K = 2, 64, 256
    wb, yb = 2 * N * K, 2 * M * N
    x0, x1 = 0x100000, 0x200000
    w0, w1 = 0x300000, 0x400000
    y0, y1 = 0x500000, 0x600000

    def ring(xs, ws, ys):
        return lib.skinny_gemm_bf16_ring(_ptrs(*xs), _ptrs(*ws), _ptrs(*ys), len(xs), M, N, K,
                                         None)

    # a chain (x of item 1 = y of item 0) is refused: the items run concurrently
    assert ring([x0, y0], [w0, w1], [y0, y1]) == sk.SKINNY_EINVAL
    assert "independent" in sk.skinny_last_error()
    assert ring([x0, x1], [w0, w1 + wb - 2], [y0, w1 + wb - 16]) == sk.SKINNY_EINVAL
    assert ring([x0, x1], [w0, w1], [y0, y0 + yb - 16]) == sk.SKINNY_EINVAL
    assert "items 0 and 1" in sk.skinny_last_error()
    assert ring([x0, None], [w0, w1], [y0, y1]) == sk.SKINNY_EINVAL
    assert "item 1" in sk.skinny_last_error()
    assert ring([x0, x1 + 8], [w0, w1], [y0, y1]) == sk.SKINNY_EINVAL
    assert "aligned" in sk.skinny_last_error()
    # one x shared by every item and disjoint outputs are fine
    assert ring([x0, x0], [w0, w1], [y0, y1]) in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)


def test_publish_reasons_without_device(sk):
    lib = ctypes.CDLL(sk.LIB_PATH)
    lib.skinny_gemm_bf16_publish.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [
        ctypes.POINTER(sk._CLaunch), ctypes.POINTER(sk._CMailbox), ctypes.c_void_p]
    M, N, K = 4, 64, 256
    x, w, y = 0x100000, 0x200000, 0x300000
    data, stage, ticket = 0x400000, 0x500000, 0x500100

    def call(data=data, stage=stage, ticket=None, tp=2, rank=1, capacity=8, width=N, launch=None):
        mb = sk._CMailbox(data, stage, ticket, tp, rank, capacity, width)
        lp = None if launch is None else ctypes.byref(sk.Launch(*launch)._c())
        return lib.skinny_gemm_bf16_publish(x, w, y, M, N, K, lp, ctypes.byref(mb), None)

    def bad(needle, **kw):
        assert call(**kw) == sk.SKINNY_EINVAL, needle
        assert needle in sk.skinny_last_error(), sk.skinny_last_error()

    bad("width 32 != N 64", width=32)
    bad("exceeds the mailbox capacity 3", capacity=3)
    bad("rank 2 of tp 2", rank=2)
    bad("rank -1 of tp 2", rank=-1)
    bad("null mailbox data", data=None)
    bad("16-byte aligned", data=data + 8)
    bad("needs a stage state or a ticket", stage=None)
    bad("4-byte aligned", stage=stage + 2)
    bad("overlaps x, W or y", data=y - 64)
    bad("overlaps the mailbox or y", stage=data + 16)
    assert lib.skinny_gemm_bf16_publish(x, w, y, M, N, K, None, None, None) == sk.SKINNY_EINVAL
    # an unsupported explicit launch is refused before the mailbox is looked at
    assert call(launch=(0, 3, 1, 1, 1, 4)) == sk.SKINNY_EUNSUPPORTED
    # valid: a stage state, or a ticket alone; both stop at the missing device
    assert call() in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)
    assert call(stage=None, ticket=ticket) in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)
    assert call(launch=(0, 1, 1, 1, 1, 4)) in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)


def test_dual_norm_reasons_without_device(sk):
    lib = ctypes.CDLL(sk.LIB_PATH)
    f = ctypes.c_float
    lib.skinny_dual_norm.argtypes = [ctypes.c_void_p] * 3 + [f, f, ctypes.c_void_p, f] + [
        ctypes.c_void_p] * 2 + [f, f, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    M, H = 4, 256
    p, r, pw, al, be, nw, o = 0x100000, 0x200000, 0x300000, 0x310000, 0x320000, 0x330000, 0x400000

    def call(p=p, r=r, pw=pw, al=al, be=be, nw=nw, o=o, M=M, H=H):
        return lib.skinny_dual_norm(p, r, pw, 1.0, 1e-6, al, 1.0, be, nw, 1.0, 1e-6, o, M, H,
                                    None)

    def bad(needle, **kw):
        assert call(**kw) == sk.SKINNY_EINVAL, needle
        assert needle in sk.skinny_last_error(), sk.skinny_last_error()

    bad("H=100", H=100)
    bad("M=0", M=0)
    bad("null pointer", be=None)
    bad("null pointer", r=None)
    bad("16-byte aligned", pw=pw + 2)
    bad("must not overlap", o=r + 16)
    bad("must not overlap", r=p + 64)
    bad("overlaps the residual or out", nw=r + 32)
    assert call() in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)
    assert call(pw=None, al=None) in (sk.SKINNY_EDEVICE, sk.SKINNY_ENOTINIT)


def test_binding_keeps_every_argument_on_one_device(sk):
    """The library computes on the current HIP device; the binding refuses
    arguments spread over several devices, and a stream of another device."""
    import torch

    class OnDevice:
        def __init__(self, d):
            self.device = torch.device(d)

    same = sk._common_device(("x", OnDevice("cuda:0")), ("W", OnDevice("cuda:0")),
                             ("ticket", None))
    assert same == torch.device("cuda:0")
    with pytest.raises(ValueError, match="one device"):
        sk._common_device(("x", OnDevice("cuda:0")), ("W", OnDevice("cuda:1")))
    with pytest.raises(ValueError, match="stream is on"):
        sk._stream(OnDevice("cuda:1"), torch.device("cuda:0"))


@pytest.mark.parametrize("name", ["skinny_ceiling_stream", "skinny_ceiling_stream_store"])
def test_ceiling_stream_argument_checks(sk, name):
    """The stream references reject bad sizes, load counts and pointers before
    touching a device."""
    from moe_decode_skinny_amd import ceiling

    lib = ctypes.CDLL(ceiling.LIB_PATH)
    fn = getattr(lib, name)
    fn.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    p = ctypes.c_void_p(4096)
    cases = [(None, 8192, 1, "null pointer"), (ctypes.c_void_p(4100), 8192, 1, "aligned"),
             (p, 8192, 3, "loads_per_lane"), (p, 8192, 2, "multiple of 16384"),
             (p, 0, 1, "positive"), (p, 1 << 31, 1, "below 2^31")]
    for src, nbytes, lpl, needle in cases:
        assert fn(src, nbytes, p, lpl, None) == sk.SKINNY_EINVAL, needle
        msg = ceiling.skinny_ceiling_last_error()
        assert needle in msg, (needle, msg)
    assert fn(p, 8192, ctypes.c_void_p(4098), 1, None) == sk.SKINNY_EINVAL


def test_last_error_is_per_thread(sk):
    """skinny_last_error is thread-local (include/skinny.h): two threads that
    fail differently, interleaved so that each failure lands between the
    other thread's failure and its read, each read back their own reason."""
    import threading

    lib = sk._lib
    step = threading.Barrier(2)
    got = {}

    def worker(name, M):
        out = sk.Launch(0, 0, 0, 0, 0, 0)._c()
        step.wait()
        if name == "a":
            assert lib.skinny_choose(M, 1024, 4096, 0, ctypes.byref(out)) == sk.SKINNY_EINVAL
            step.wait()  # b fails now
            step.wait()
        else:
            step.wait()
            assert lib.skinny_choose(M, 1024, 4096, 0, ctypes.byref(out)) == sk.SKINNY_EINVAL
            step.wait()
        got[name] = lib.skinny_last_error().decode()

    ts = [threading.Thread(target=worker, args=("a", 17)), threading.Thread(target=worker, args=("b", 0))]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=30)
    assert "M=17" in got["a"] and "M=0" in got["b"], got
