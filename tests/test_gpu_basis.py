"""GPU parity of the randomised Cholesky-QR basis fit (lowram_fit_basis).

Both sides take the same bf16 keys and the same bf16 Gaussian test matrix.
The fit is unique only as a subspace where the spectrum has a gap (the
synthetic keys' 64-dimensional latent part); inside the noise part, any
rounding rotates the basis.  So the comparison is on what is unique:
  - orthonormal rows (up to the bf16 storage of the basis);
  - the latent subspace contained: its largest principal angle to the GPU
    basis within a few times that of the oracle's fit rounded to bf16;
  - the projection error of the keys within 1% of the oracle fit's (rounded
    to bf16), and never below the exact SVD optimum (small cases);
  - status 0 (every Cholesky pivot positive).
For a given test matrix the fit is also unique as a basis: Cholesky-QR with
a positive-diagonal R fixes every row's sign.  So the GPU basis is compared
with the oracle's directly as well:
  - all r principal angles between the two spans;
  - the entries, row by row after aligning each row's sign.
The bounds are about three times what the GPU's roundings give in a numpy
emulation of them (fp32 products, bf16 intermediates, bf16 output): at c0
sizes the largest angle 0.002-0.021 rad and the largest entry difference
0.0005-0.0033; at the 32K size 0.056 rad and 0.0034.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from gpu_util import DEV, up  # noqa: E402
from long_context_decode_landmark_amd import native  # noqa: E402
from oracle import basis, codecs  # noqa: E402


def host16(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def run_fit(x_bits, om_t_bits, rank, power):
    nb, T, D = x_bits.shape
    P = om_t_bits.shape[-1]
    shape = native.fit_shape(nb, T, P, D, rank, power)
    ws = torch.empty(native.fit_basis_workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    out = torch.zeros((nb, rank, D), dtype=torch.int16, device=DEV)
    status = torch.full((nb,), -1, dtype=torch.int32, device=DEV)
    native.fit_basis(shape, up(x_bits), up(om_t_bits), out, status, ws)
    torch.cuda.synchronize()
    return codecs.bf16_decode(host16(out)), status.cpu().numpy()


def compare_bases(b_g, b_or, angle_tol, entry_tol, what):
    """All principal angles between the spans, and the sign-aligned entries."""
    ang = float(np.max(basis.principal_angles(b_or, b_g)))
    sign = np.sign(np.sum(b_or * b_g, axis=1))[:, None]
    ent = float(np.max(np.abs(b_or - sign * b_g)))
    print(f"{what}: largest of {len(b_or)} principal angles to the oracle's basis {ang:.1e} rad, "
          f"largest sign-aligned entry difference {ent:.1e}", flush=True)
    assert np.all(sign != 0)
    assert ang <= angle_tol, (what, ang)
    assert ent <= entry_tol, (what, ent)


def latent_rows(cfg, b, grp):
    """Orthonormal rows spanning the keys' latent subspace (row space of the mixing matrix)."""
    q, _ = np.linalg.qr(synth.draws.mixing(cfg, b, grp).T)
    return q.T


@pytest.mark.parametrize("name,cfg,power", [
    ("c0_r64_p1", synth.C0, 1),
    ("c0_r128_p1", synth.C0.with_(name="fitg", rank=128), 1),
    ("c0_r128_p0", synth.C0.with_(name="fitg0", rank=128), 0),
    ("c0_r256_p2_b2", synth.C0.with_(name="fitg2", rank=256, batch=2), 2),
])
def test_fit_matches_oracle(name, cfg, power):
    P, r = cfg.prefix, cfg.rank
    rng = np.random.default_rng(31)
    xs = [codecs.bf16_encode(synth.exact_keys(cfg, b, 0)) for b in range(cfg.batch)]
    oms = [codecs.bf16_encode(rng.standard_normal((r, P))) for _ in range(cfg.batch)]
    got, status = run_fit(np.stack(xs), np.stack(oms), r, power)
    assert np.all(status == 0), status
    for b in range(cfg.batch):
        x = codecs.bf16_decode(xs[b][:P])
        b_or = basis.randomized_cholqr(x, codecs.bf16_decode(oms[b]).T, power=power)
        b_or16 = codecs.bf16_round(b_or)
        b_g = got[b]
        ortho = float(np.max(np.abs(b_g @ b_g.T - np.eye(r))))
        ortho_ref = float(np.max(np.abs(b_or16 @ b_or16.T - np.eye(r))))
        assert ortho <= 4 * ortho_ref + 1e-3, (ortho, ortho_ref)
        lat = latent_rows(cfg, b, 0)
        a_g, a_ref = basis.max_angle(lat, b_g), basis.max_angle(lat, b_or16)
        assert a_g <= 4 * a_ref + 2e-3, (a_g, a_ref)
        e_g, e_ref = basis.projection_error(x, b_g), basis.projection_error(x, b_or16)
        e_svd = basis.projection_error(x, basis.svd_basis(x, r))
        assert abs(e_g - e_ref) <= 1e-2 * e_ref, (e_g, e_ref)
        assert e_g >= e_svd * (1 - 1e-3)
        compare_bases(b_g, b_or, 0.06, 0.01, f"fit {name} b{b}")
        print(f"\nfit {name} b{b}: ortho {ortho:.1e} (ref {ortho_ref:.1e}) latent angle {a_g:.1e} "
              f"(ref {a_ref:.1e}) proj err {e_g:.4f} (ref {e_ref:.4f}, svd {e_svd:.4f})", flush=True)


def test_fit_c1_size():
    """32640 tokens x 4096 key dims, rank 512, one power pass."""
    cfg, power = synth.C1, 1
    P, r = cfg.prefix, cfg.rank
    x_bits = codecs.bf16_encode(synth.exact_keys(cfg, 0, 0, dtype=np.float32))
    om = codecs.bf16_encode(np.random.default_rng(32).standard_normal((r, P)))
    got, status = run_fit(x_bits[None], om[None], r, power)
    assert status[0] == 0
    x = codecs.bf16_decode(x_bits[:P])
    b_or16 = codecs.bf16_round(basis.randomized_cholqr(x, codecs.bf16_decode(om).T, power=power))
    b_g = got[0]
    lat = latent_rows(cfg, 0, 0)
    a_g, a_ref = basis.max_angle(lat, b_g), basis.max_angle(lat, b_or16)
    e_g, e_ref = basis.projection_error(x, b_g), basis.projection_error(x, b_or16)
    ortho = float(np.max(np.abs(b_g @ b_g.T - np.eye(r))))
    print(f"\nfit c1: ortho {ortho:.1e} latent angle {a_g:.1e} (ref {a_ref:.1e}) proj err {e_g:.5f} (ref {e_ref:.5f})",
          flush=True)
    assert ortho <= 2e-2
    assert a_g <= 4 * a_ref + 2e-3
    assert abs(e_g - e_ref) <= 1e-2 * e_ref
    compare_bases(b_g, basis.randomized_cholqr(x, codecs.bf16_decode(om).T, power=power), 0.17, 0.012, "fit c1")


def test_fit_full_size_properties():
    """The 262K group of the benchmark (device-drawn keys): orthonormal rows,
    the latent subspace contained, and the projection error of sampled tokens
    close to the noise floor (the keys' non-latent energy)."""
    from synth import device as sd
    cfg = synth.C3
    P, r, D = cfg.prefix, cfg.rank, cfg.group_dim
    d_in = sd.draw_build_inputs(cfg, 99, DEV, 1, layers=[])
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    om = torch.randn((1, r, P), generator=g, device=DEV).to(torch.bfloat16)
    shape = native.fit_shape(1, cfg.ctx, P, D, r, 1)
    ws = torch.empty(native.fit_basis_workspace_bytes(shape), dtype=torch.uint8, device=DEV)
    out = torch.zeros((1, r, D), dtype=torch.int16, device=DEV)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    native.fit_basis(shape, d_in["keys"], om, out, status, ws)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    b_g = codecs.bf16_decode(host16(out)[0])
    ortho = float(np.max(np.abs(b_g @ b_g.T - np.eye(r))))
    a_g = basis.max_angle(latent_rows(cfg, 0, 0), b_g)
    idx = np.random.default_rng(3).choice(P, 4096, replace=False)
    x = codecs.bf16_decode(host16(d_in["keys"][0])[idx])
    e_g = basis.projection_error(x, b_g)
    # the best any rank-512 basis can do on noise of std 0.05 in 4096 - 64 latent-free dims
    floor = 0.05 * np.sqrt((D - r) / 1.0) / np.sqrt(np.mean(np.sum(x * x, axis=1)))
    print(f"\nfit c3: ortho {ortho:.1e} latent angle {a_g:.1e} proj err {e_g:.4f} (noise floor ~{floor:.4f})",
          flush=True)
    assert ortho <= 2e-2
    assert a_g <= 1e-2
    assert e_g <= 1.2 * floor
