"""The C ABI: the library loads without a GPU, exports every function the
header declares, and its host-side validation and variant choice behave as
documented.  No kernel is launched here (every call below is rejected or is
a no-op before any HIP call)."""
import ctypes
import os
import re

import pytest

import barrier_pipelined_tiled_amd as pkg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bpt_gemm.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pkg.LIB_PATH):
        from barrier_pipelined_tiled_amd import build
        build.build()
    return pkg.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("gemm_f16", "gemm_bf16", "gemm_batched_f16", "gemm_ex", "bpt_status_string",
              "bpt_last_error", "bpt_variant_count", "bpt_variant_name", "bpt_select_variant"):
        assert f in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in bpt_gemm.h but not exported"


def test_the_poison_build_exports_the_same_boundary():
    """The race-detection build (every LDS-DMA destination NaN-filled before
    its copy) is the same library: it loads without a GPU, exports every
    declared function and has the same variant table."""
    if not os.path.exists(pkg.POISON_LIB_PATH):
        from barrier_pipelined_tiled_amd import build
        build.build_poison()
    normal = pkg.variants()
    with pkg.library(pkg.POISON_LIB_PATH) as P:
        for name in declared_functions():
            assert hasattr(P, name), f"{name} not exported by the poison build"
        assert pkg.variants() == normal
    assert pkg.lib() is not P


def test_no_torch_types_in_header():
    text = open(HEADER).read()
    assert "at::Tensor" not in text and "c10" not in text


def test_status_strings(L):
    assert L.bpt_status_string(0) == b"BPT_OK"
    assert L.bpt_status_string(1) == b"BPT_ERR_INVALID_ARG"
    assert L.bpt_status_string(2) == b"BPT_ERR_UNSUPPORTED"
    assert L.bpt_status_string(3) == b"BPT_ERR_HIP"


def test_variant_table(L):
    names = pkg.variants()
    assert len(names) == L.bpt_variant_count() >= 3
    assert L.bpt_variant_name(0) is None and L.bpt_variant_name(L.bpt_variant_count() + 1) is None
    assert "generic_64x64x16" in names
    assert any(n.startswith("pipelined_256x256x64") for n in names)


FAKE = 1 << 20          # a 16-byte aligned non-null address; never dereferenced below


@pytest.mark.parametrize("args,what", [
    ((-1, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 0), "negative M"),
    ((4, -1, 4, FAKE, 4, FAKE, 4, FAKE, 4, 0), "negative N"),
    ((4, 4, -1, FAKE, 4, FAKE, 4, FAKE, 4, 0), "negative K"),
    ((4, 4, 8, FAKE, 7, FAKE, 4, FAKE, 4, 0), "lda < K"),
    ((4, 8, 4, FAKE, 4, FAKE, 7, FAKE, 8, 0), "ldb < N"),
    ((4, 8, 4, FAKE, 4, FAKE, 8, FAKE, 7, 0), "ldc < N"),
    ((4, 4, 4, FAKE, 4, FAKE, 4, FAKE, 4, 2), "out_fp32 not 0/1"),
    ((4, 4, 4, 0, 4, FAKE, 4, FAKE, 4, 0), "A NULL"),
    ((4, 4, 4, FAKE, 4, 0, 4, FAKE, 4, 0), "B NULL"),
    ((4, 4, 4, FAKE, 4, FAKE, 4, 0, 4, 0), "C NULL"),
])
def test_invalid_arguments_rejected(L, args, what):
    for fn in (L.gemm_f16, L.gemm_bf16):
        st = fn(*args, None)
        assert st == pkg.BPT_ERR_INVALID_ARG, what
        assert L.bpt_last_error().decode() != ""


def test_batched_invalid(L):
    st = L.gemm_batched_f16(-1, 4, 4, 4, FAKE, 4, 16, FAKE, 4, 16, FAKE, 4, 16, 0, None)
    assert st == pkg.BPT_ERR_INVALID_ARG
    st = L.gemm_batched_f16(2, 4, 4, 4, FAKE, 4, -16, FAKE, 4, 16, FAKE, 4, 16, 0, None)
    assert st == pkg.BPT_ERR_INVALID_ARG
    st = L.gemm_ex(2, 1, 4, 4, 4, FAKE, 4, 0, FAKE, 4, 0, FAKE, 4, 0, 0, 0, None)
    assert st == pkg.BPT_ERR_INVALID_ARG          # dtype 2 does not exist
    st = L.gemm_ex(0, 1, 4, 4, 4, FAKE, 4, 0, FAKE, 4, 0, FAKE, 4, 0, 0, 99, None)
    assert st == pkg.BPT_ERR_INVALID_ARG          # no variant 99


def test_oversized_dimension_unsupported(L):
    big = 1 << 31
    st = L.gemm_f16(4, big, 4, FAKE, 4, FAKE, big, FAKE, big, 0, None)
    assert st == pkg.BPT_ERR_UNSUPPORTED


def test_empty_shapes_are_noops(L):
    # nothing to compute: OK with no launch (NULL pointers allowed)
    assert L.gemm_f16(0, 16, 16, 0, 16, 0, 16, 0, 16, 0, None) == pkg.BPT_OK
    assert L.gemm_f16(16, 0, 16, 0, 16, 0, 1, 0, 1, 0, None) == pkg.BPT_OK
    assert L.gemm_batched_f16(0, 16, 16, 16, 0, 16, 0, 0, 16, 0, 0, 16, 0, 0, None) == pkg.BPT_OK


def test_apair_variant_requirements(L):
    """The A-pair kernel reads A in 64-wide K pairs with a 4-stage B ring:
    K must be a multiple of 64 and at least 192; no K tail."""
    v = pkg.variants()["pipelined_256x256x32_s4_apair"]
    for K in (64, 128, 96, 200, 4104):
        st = L.gemm_ex(0, 1, 256, 256, K, FAKE, K, 0, FAKE, 256, 0, FAKE, 256, 0, 0, v, None)
        assert st == pkg.BPT_ERR_UNSUPPORTED, K
    # B given transposed is not its layout
    st = L.gemm_ex_bt(0, 1, 256, 256, 256, FAKE, 256, 0, FAKE, 256, 0, FAKE, 256, 0, 0, v, None)
    assert st == pkg.BPT_ERR_UNSUPPORTED


def test_forced_variant_that_cannot_take_the_call(L):
    v = pkg.variants()["pipelined_256x256x64_s2"]
    # K = 100 is not a multiple of the 64-wide K-tile
    st = L.gemm_ex(0, 1, 256, 256, 100, FAKE, 100, 0, FAKE, 256, 0, FAKE, 256, 0, 0, v, None)
    assert st == pkg.BPT_ERR_UNSUPPORTED
    # unaligned A
    st = L.gemm_ex(0, 1, 256, 256, 128, FAKE + 2, 128, 0, FAKE, 256, 0, FAKE, 256, 0, 0, v, None)
    assert st == pkg.BPT_ERR_UNSUPPORTED


def test_automatic_variant_choice():
    v = pkg.variants()
    big = v["pipelined_256x256x32_s4"]
    # K a multiple of 64 (and >= 192): A copied in K-tile pairs, whole lines
    apair = v["pipelined_256x256x32_s4_apair"]
    assert pkg.select_variant("f16", 1, 4096, 4096, 4096, 4096, 4096) == apair
    assert pkg.select_variant("bf16", 1, 4096, 4096, 16384, 16384, 4096, True) == apair
    # short K over >= 256 row blocks of 128 and >= 2048 tiles of 128 x 256
    # (16-bit C): the persistent kernel with wave roles, K = 256 and 128
    roles = v["persistent_128x256x32_shortk_roles"]
    assert pkg.select_variant("f16", 64, 4096, 4096, 256, 256, 4096) == roles
    assert pkg.select_variant("bf16", 64, 4096, 4096, 128, 128, 4096) == roles
    assert pkg.select_variant("f16", 8, 4096, 4096, 256, 256, 4096) == roles
    # fewer row blocks, >= 2048 tiles of 256 x 128: the A-pair persistent kernel,
    # at K = 128 the one keeping each row block's A panel in LDS
    persist = v["persistent_256x128x32_shortk_apair"]
    assert pkg.select_variant("f16", 4, 4096, 4096, 256, 256, 4096) == persist
    assert pkg.select_variant("f16", 4, 4096, 4096, 128, 128, 4096) == v["persistent_256x128x32_shortk_aresident"]
    # N not a multiple of 256: the A-pair persistent kernel
    assert pkg.select_variant("f16", 64, 4096, 4224, 256, 256, 4224) == persist
    assert pkg.select_variant("f16", 2, 4096, 4096, 256, 256, 4096) == apair      # 1024 tiles
    assert pkg.select_variant("f16", 64, 4096, 4096, 256, 256, 4096, True) == apair   # fp32 C
    assert pkg.select_variant("f16", 64, 4096, 4096, 192, 192, 4096) == apair     # K not 128 or 256
    assert pkg.select_variant("f16", 1, 4096, 4096, 192, 192, 4096) == apair
    # K = 160 (five 32-wide tiles): too short for the pair ring, the 4-stage kernel
    assert pkg.select_variant("f16", 1, 4096, 4096, 160, 160, 4096) == big
    assert pkg.select_variant("f16", 1, 256, 256, 256, 256, 256) == v["pipelined_128x128x32_s4"]
    # K = 96: three 32-wide tiles (< 4 stages) and not a multiple of 64
    assert pkg.select_variant("f16", 1, 256, 256, 96, 96, 256) == v["generic_64x64x16"]
    # K = 128: four 32-wide tiles fill the four-stage ring
    assert pkg.select_variant("f16", 1, 4096, 4096, 128, 128, 4096) == big
    # K = 200 = 6 x 32 + 8: six full K-tiles and a partial one in its own stage
    assert pkg.select_variant("f16", 1, 256, 256, 200, 200, 256) == v["pipelined_128x128x32_s4"]
    assert pkg.select_variant("f16", 1, 4096, 4096, 4104, 4104, 4096) == big
    # K % 8 != 0 (a chunk of A would straddle K), odd leading dimension,
    # unaligned base: no pipelined kernel reads them in place.  From 2^24
    # multiply-adds on they are copied, zero-padded and aligned, into a
    # workspace first (256^3 is exactly 2^24); smaller ones take the guarded
    # kernel
    repack = v["repack_pipelined"]
    assert pkg.select_variant("f16", 1, 256, 256, 196, 196, 256) == v["generic_64x64x16"]
    assert pkg.select_variant("f16", 1, 256, 256, 256, 260, 257) == repack
    assert pkg.select_variant("f16", 1, 256, 256, 256, 256, 256, A_ptr=FAKE + 2) == repack
    assert pkg.select_variant("f16", 1, 4096, 4096, 4090, 4090, 4096) == repack
    assert pkg.select_variant("f16", 1, 100, 70, 50, 50, 70) == v["generic_64x64x16"]
    # K = 64 is one 64-wide tile (two stages need two) and two 32-wide tiles
    # (four stages need four)
    assert pkg.select_variant("f16", 1, 256, 256, 64, 64, 256) == v["generic_64x64x16"]
    # few rows of A: the shared-ring skinny kernel (128-column blocks, K
    # split over up to 64 workgroups to reach one workgroup per CU), for any K
    # that is a multiple of 32 ...
    ring = v["skinny_64x128_ring_k32_s4_splitk"]
    wide, narrow = v["skinny_64x128_w4_k32_s4_splitk"], v["skinny_64x32_w4_k64_s4"]
    assert pkg.select_variant("f16", 1, 64, 8192, 8192, 8192, 8192) == ring
    assert pkg.select_variant("f16", 1, 16, 4096, 4096, 4096, 4096) == ring
    assert pkg.select_variant("f16", 1, 1, 32768, 512, 512, 32768) == ring      # 256 blocks, no split
    assert pkg.select_variant("f16", 1, 64, 4096, 1024, 1024, 4096) == ring     # 32 blocks x 8 splits
    assert pkg.select_variant("f16", 1, 64, 8192, 768, 768, 8192) == ring       # 64 blocks x 4 splits
    assert pkg.select_variant("f16", 1, 64, 16384, 96, 96, 16384) == ring       # 3 chunks, no split
    # narrow outputs over long K: fewer than 128 workgroups either way, but
    # the ring's K splits give more than the output tiles
    assert pkg.select_variant("f16", 1, 64, 512, 65536, 65536, 512) == ring      # 4 blocks x 8 against 4 tiles
    assert pkg.select_variant("f16", 1, 64, 256, 8192, 8192, 256) == ring        # 2 x 8 against 2
    # ... but not when the output tiles already fill the chip
    assert pkg.select_variant("f16", 64, 100, 4096, 256, 256, 4096) != ring
    # up to 128 rows (two row blocks) while 128 x 128 tiles would leave CUs
    # idle; from 129 rows, or with 256 or more such tiles, the pipelined kernels
    assert pkg.select_variant("f16", 1, 128, 8192, 8192, 8192, 8192) == ring
    assert pkg.select_variant("f16", 1, 96, 8192, 8192, 8192, 8192) == ring
    assert pkg.select_variant("f16", 1, 128, 4096, 4096, 4096, 4096) == ring
    splitk = v["splitk_pipelined"]
    assert pkg.select_variant("f16", 1, 129, 8192, 8192, 8192, 8192) == splitk
    assert pkg.select_variant("f16", 1, 192, 8192, 8192, 8192, 8192) == splitk
    assert pkg.select_variant("f16", 1, 128, 32768, 4096, 4096, 32768) == v["pipelined_256x256x32_s4_apair"]
    # ... which makes the other two skinny kernels forced-only: each needs
    # K a multiple of 256 or more, where the ring fits at least as many
    # splits
    assert pkg.select_variant("f16", 1, 64, 8192, 8200, 8200, 8192) not in (ring, wide, narrow)
    # N % 8 != 0: column chunks would straddle N in place, so the operands are
    # repacked (B to a width of 8192 resp. 4096, C stored at the true N)
    assert pkg.select_variant("f16", 1, 64, 8190, 8192, 8192, 8190) == repack
    assert pkg.select_variant("f16", 1, 4096, 4092, 4096, 4096, 4092) == repack
    # ... unless K is too short for any ring even after padding
    assert pkg.select_variant("f16", 1, 4096, 4092, 96, 96, 4092) == v["generic_64x64x16"]
    # split-K: at most 128 tiles of 128 x 128 leave half the CUs idle, so K
    # is split over the pipelined kernel's batch (2 to 64 ranges, each a
    # multiple of 64 and at least 256 long, tiles x splits <= 256)
    assert pkg.select_variant("f16", 1, 256, 8192, 8192, 8192, 8192) == splitk    # 128 tiles x 2
    assert pkg.select_variant("f16", 1, 1024, 1024, 8192, 8192, 1024) == splitk   # 64 tiles x 4
    assert pkg.select_variant("bf16", 1, 512, 512, 4096, 4096, 512, True) == splitk  # 16 tiles x 8
    assert pkg.select_variant("f16", 1, 384, 8192, 8192, 8192, 8192) == v["pipelined_128x128x32_s4"]  # 192 tiles
    assert pkg.select_variant("f16", 1, 256, 8192, 384, 384, 8192) == v["pipelined_128x128x32_s4"]    # K/2 < 256
    assert pkg.select_variant("f16", 2, 256, 8192, 8192, 8192, 8192) not in (splitk, 0)                # batched
    assert pkg.select_variant("f16", 1, 256, 8192, 8200, 8200, 8192) != splitk    # K not a multiple of 128
    # rejected / nothing to do
    assert pkg.select_variant("f16", 1, 0, 256, 256, 256, 256) == 0
    assert pkg.select_variant("f16", 1, 16, 16, 16, 8, 16) == 0


def test_bt_layout_entry_point(L):
    """gemm_ex_bt: Bt's leading dimension is checked against K, and each
    layout rejects the other's forced variants (no launch happens)."""
    v = pkg.variants()
    # ldbt < K
    st = L.gemm_ex_bt(0, 1, 64, 64, 128, FAKE, 128, 0, FAKE, 100, 0, FAKE, 64, 0, 0, 0, None)
    assert st == pkg.BPT_ERR_INVALID_ARG
    # ldbt >= K but < N is fine for this layout; a B-as-K x N variant is not
    st = L.gemm_ex_bt(0, 1, 256, 512, 128, FAKE, 128, 0, FAKE, 128, 0, FAKE, 512, 0, 0,
                      v["pipelined_256x256x32_s4"], None)
    assert st == pkg.BPT_ERR_UNSUPPORTED
    st = L.gemm_ex(0, 1, 256, 256, 128, FAKE, 128, 0, FAKE, 256, 0, FAKE, 256, 0, 0,
                   v["pipelined_bt_256x256x32_s4"], None)
    assert st == pkg.BPT_ERR_UNSUPPORTED
    # automatic choice for the transposed layout
    # A in whole-line K-tile pairs when K % 64 == 0 and K >= 192 ...
    assert pkg.select_variant("f16", 1, 4096, 4096, 4096, 4096, 4096, bt=True) == v["pipelined_bt_256x256x32_s4_apair"]
    # ... and N need not be a multiple of 8 here
    assert pkg.select_variant("f16", 1, 4096, 4095, 4096, 4096, 4096, bt=True) == v["pipelined_bt_256x256x32_s4_apair"]
    # K = 128: too short for the pairs, 64-wide K-tiles (whole 128-byte rows) in 2 stages
    assert pkg.select_variant("f16", 1, 4096, 4096, 128, 128, 128, bt=True) == v["pipelined_bt_256x256x64_s2"]
    # K = 4104: no 64-wide tiling, the 32-wide one with a tail
    assert pkg.select_variant("f16", 1, 4096, 4096, 4104, 4104, 4104, bt=True) == v["pipelined_bt_256x256x32_s4"]
    assert pkg.select_variant("f16", 1, 256, 200, 256, 256, 256, bt=True) == v["pipelined_bt_128x128x32_s4"]
    # odd K and odd leading dimensions: the guarded kernel
    assert pkg.select_variant("f16", 1, 300, 201, 250, 250, 250, bt=True) == v["generic_bt_64x64x16"]
    # few output tiles: split-K, as for the other layout (N a multiple of 8)
    assert pkg.select_variant("f16", 1, 256, 8192, 8192, 8192, 8192, bt=True) == v["splitk_pipelined"]
    assert pkg.select_variant("f16", 1, 256, 8190, 8192, 8192, 8192, bt=True) == v["pipelined_bt_128x128x32_s4"]



def _attn(L, dtype=0, BH=2, Sq=128, Skv=64, D=256, Q=FAKE, ldq=256, sQ=0, K=FAKE, ldk=256, sK=0,
          V=FAKE, ldv=256, sV=0, O=FAKE, ldo=256, sO=0, scale=0.0625, out_fp32=0):
    return L.attention_fwd(dtype, BH, Sq, Skv, D, Q, ldq, sQ, K, ldk, sK, V, ldv, sV, O, ldo, sO,
                           scale, out_fp32, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), pkg.BPT_ERR_INVALID_ARG),
    (dict(out_fp32=3), pkg.BPT_ERR_INVALID_ARG),
    (dict(BH=-1), pkg.BPT_ERR_INVALID_ARG),
    (dict(Sq=-1), pkg.BPT_ERR_INVALID_ARG),
    (dict(Skv=-1), pkg.BPT_ERR_INVALID_ARG),
    (dict(D=0), pkg.BPT_ERR_INVALID_ARG),
    (dict(ldq=128), pkg.BPT_ERR_INVALID_ARG),
    (dict(ldk=255), pkg.BPT_ERR_INVALID_ARG),
    (dict(ldv=8), pkg.BPT_ERR_INVALID_ARG),
    (dict(ldo=200), pkg.BPT_ERR_INVALID_ARG),
    (dict(sV=-8), pkg.BPT_ERR_INVALID_ARG),
    (dict(scale=float("nan")), pkg.BPT_ERR_INVALID_ARG),
    (dict(scale=float("inf")), pkg.BPT_ERR_INVALID_ARG),
    (dict(Q=0), pkg.BPT_ERR_INVALID_ARG),
    (dict(O=0), pkg.BPT_ERR_INVALID_ARG),
    (dict(K=0), pkg.BPT_ERR_INVALID_ARG),
    (dict(V=0), pkg.BPT_ERR_INVALID_ARG),
    (dict(D=64, ldq=64, ldk=64, ldv=64, ldo=64), pkg.BPT_ERR_UNSUPPORTED),     # head_dim not built
    (dict(D=96, ldq=96, ldk=96, ldv=96, ldo=96), pkg.BPT_ERR_UNSUPPORTED),
    (dict(Q=FAKE + 8), pkg.BPT_ERR_UNSUPPORTED),                              # 8-byte aligned base
    (dict(ldk=260), pkg.BPT_ERR_UNSUPPORTED),                                 # row not 16-byte granular
    (dict(sO=12), pkg.BPT_ERR_UNSUPPORTED),
    (dict(Skv=1 << 22, ldk=256), pkg.BPT_ERR_UNSUPPORTED),                     # head's K extent >= 2^31 bytes
    (dict(Skv=4194240), pkg.BPT_ERR_UNSUPPORTED),          # the first Skv whose K (+64 rows) reaches 2^31 bytes
])
def test_attention_rejections(L, kw, status):
    assert _attn(L, **kw) == status, kw
    assert L.bpt_last_error().decode() != ""


def test_attention_empty_calls_are_noops(L):
    # nothing to compute: OK, no launch, NULL pointers allowed
    assert _attn(L, BH=0, Q=0, K=0, V=0, O=0) == pkg.BPT_OK
    assert _attn(L, Sq=0, Q=0, K=0, V=0, O=0) == pkg.BPT_OK


def test_noalloc_rejects_a_call_needing_more_scratch(L):
    """The no-allocation entry point refuses, before any launch, a call whose
    path needs more scratch than its fixed array: 4096 x 4095 x 4090 takes
    the repack route, whose padded copies of A and B need 64 MiB."""
    assert L.bpt_noalloc_scratch_bytes() == 32 << 20
    M, N, K = 4096, 4095, 4090
    FAKEP = 1 << 20
    st = L.gemm_ex_noalloc(0, 1, M, N, K, FAKEP, K, 0, FAKEP, N, 0, FAKEP, N, 0, 0, 0, None)
    assert st == pkg.BPT_ERR_UNSUPPORTED
    msg = L.bpt_last_error().decode()
    assert "scratch" in msg and str(32 << 20) in msg
