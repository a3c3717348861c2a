"""The achievable-rate probes (mpq_probe_rate) run and read plausibly: every
rate positive and at most 10 % above the MI355X figure it is read against
(the probes reach, not exceed, the hardware's rates)."""
import pytest

pytestmark = pytest.mark.gpu

VENDOR = {"mfma_bf16": 2.5e15, "mfma_f64": 78.6e12, "valu_f64": 78.6e12, "exp_f32": 256 * 4 * 16 * 2.4e9,
          "hbm_copy": 8.0e12, "mfma_i8": 5.0e15}


@pytest.mark.parametrize("kind", sorted(VENDOR))
def test_probe_rate(kind):
    import torch
    import post_quantization_solver_amd as mpq
    # the copy streams 1 GiB each way, four times the 256 MB last-level cache
    scratch = torch.empty((2 << 30) if kind == "hbm_copy" else (8 << 20), dtype=torch.uint8, device="cuda")
    rate = mpq.probe_rate(kind, scratch)
    print(f"[probe] {kind}: {rate:.4g} ({rate / VENDOR[kind]:.2f} of the vendor figure)", flush=True)
    assert 0.0 < rate <= 1.1 * VENDOR[kind]
