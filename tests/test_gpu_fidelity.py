"""The fidelity report's GPU leg: the kernel's output against exact fp64
attention on the unquantized fp32 inputs.

Page 1's KLD tables (q4_0 V and q8_0 V against fp16 V) measure what the
packed formats cost end to end.  oracle/fidelity.py measures the same costs
at the kernel level on the workload inputs, for the oracle's arithmetic.
Here the HIP output enters the same report: its relative L2 distance to the
exact attention must equal the oracle's int8-Q.K column for the matching V
format to within the parity tolerance (the kernel adds its own fp32/fp16
rounding, which is at most 1e-3 of the output, on top of the formats' 0.5-9%).
The lines printed with -s are the GPU column of the report."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from decode_attention_packed_amd import workloads as W  # noqa: E402
from oracle import fidelity as F  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402


@pytest.mark.parametrize("name,fmt,kv_heads", [("tiny", W.V_Q4_0, None), ("gqa8k", W.V_Q4_0, None),
                                               ("gqa8k", W.V_Q8_0, None),
                                               ("long128k", W.V_Q4_0, [0, 5])])
def test_kernel_error_equals_format_error(name, fmt, kv_heads):
    ci = [c for c in W.make_inputs(name) if c.spec.v_format == fmt][0]
    spec = ci.spec
    print(f"[gpu-test] fidelity {spec.name}", flush=True)
    cache, table, max_segs = H.build_cache(ci)
    got = H.run_attention(cache, ci, table, max_segs)[0]          # [Tq][Hq][D]
    del cache
    L = int(ci.seq_len[0])
    q, k, v = ci.q[0], ci.k[0][:L], ci.v[0][:L]
    rep = F.workload_report(q, k, v, spec.sm_scale, kv_heads)
    fmt_name = "q4_0" if fmt == W.V_Q4_0 else "q8_0"
    e_oracle = float(rep["rel_l2"][("int8", fmt_name)])
    e_gpu = F.output_error(q, k, v, spec.sm_scale, got, kv_heads)
    heads = "all" if kv_heads is None else f"kv heads {kv_heads}"
    print(f"[fidelity-gpu] {spec.name} ({L} tokens, {heads}): out rel-L2 vs exact: kernel "
          f"{e_gpu:.4e}, oracle int8 Q.K + {fmt_name} V {e_oracle:.4e}, f16 Q.K + {fmt_name} V "
          f"{float(rep['rel_l2'][('f16', fmt_name)]):.4e}", flush=True)
    # ||gpu - exact|| and ||oracle - exact|| differ by at most ||gpu - oracle||,
    # which parity bounds by 1e-3 of ||oracle|| (about ||exact||)
    assert abs(e_gpu - e_oracle) <= H.RTOL_L2 * (1.0 + e_oracle)
    assert np.isfinite(e_gpu)
