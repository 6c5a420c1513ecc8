"""Child process of test_debug_mode_rejects_corrupt_offsets (run with
FA_DEBUG=1): valid packed offsets run normally, corrupt ones are refused with
FA_ERR_SEQLENS before any attention kernel runs.  Every offset stays inside
the 200-token buffers."""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main() -> int:
    import numpy as np
    import torch

    import exact_io_aware_amd as fa
    from exact_io_aware_amd import _lib
    assert os.environ.get("FA_DEBUG") == "1"
    dev = "cuda:0"
    T, Hq, Hkv, d, N = 200, 4, 2, 128, 120
    gen = torch.Generator(device="cpu").manual_seed(5)
    q, k, v = (torch.randn(T, h, d, generator=gen).to(torch.bfloat16).to(dev)
               for h in (Hq, Hkv, Hkv))
    S = _lib.STATUS
    cases = [("valid", [0, 100, 200], "FA_OK"),
             ("first offset not 0", [5, 100, 200], "FA_ERR_SEQLENS"),
             ("decreasing", [0, 120, 100], "FA_ERR_SEQLENS"),
             ("length above N", [0, 60, 200], "FA_ERR_SEQLENS")]
    scale = d ** -0.5
    for label, offs, want in cases:
        print(f"case {label}: {offs}", flush=True)
        cu = torch.tensor(offs, dtype=torch.int32, device=dev)
        B = len(offs) - 1
        for entry in ("fa_fwd", "fa_fwd_kv", "fa_fwd_kv_split", "fa_fwd_sparse", "fa_bwd"):
            o = torch.full((T, Hq, d), float("nan"), device=dev)
            lse = torch.full((B, Hq, N), float("nan"), device=dev)
            torch.cuda.synchronize()
            st_ = torch.cuda.current_stream().cuda_stream
            a = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
            if entry == "fa_fwd":
                st = _lib.fwd_raw(*a, B, Hq, Hkv, N, d, 1, scale, cu.data_ptr(), st_,
                                  fa.FA_BF16, fa.FA_F32)
            elif entry == "fa_fwd_kv":
                st = _lib.fwd_kv_raw(*a, B, Hq, Hkv, N, N, d, 1, scale, cu.data_ptr(),
                                     cu.data_ptr(), st_, fa.FA_BF16, fa.FA_F32)
            elif entry == "fa_fwd_kv_split":
                part = torch.empty(fa.split_workspace_bytes(B, Hq, N, d, 2), dtype=torch.uint8,
                                   device=dev)
                st = _lib.fwd_kv_split_raw(*a, B, Hq, Hkv, N, N, d, 1, scale, cu.data_ptr(),
                                           cu.data_ptr(), 2, part.data_ptr(), part.numel(), st_,
                                           fa.FA_BF16, fa.FA_F32)
            elif entry == "fa_fwd_sparse":
                nb = -(-N // 64)
                bm = torch.ones((1, 1, nb, nb), dtype=torch.uint8, device=dev)
                st = _lib.fwd_sparse_raw(*a, B, Hq, Hkv, N, N, d, 1, scale, cu.data_ptr(),
                                         cu.data_ptr(), bm.data_ptr(), 1, 1, st_, fa.FA_BF16,
                                         fa.FA_F32)
            else:
                if want == "FA_OK":
                    continue            # the valid backward is covered by its own tests
                ob = torch.zeros((T, Hq, d), dtype=torch.bfloat16, device=dev)
                lz = torch.zeros((B, Hq, N), device=dev)
                ws = torch.empty(fa.bwd_workspace_bytes(B, Hq, Hkv, N, d, fa.FA_BF16),
                                 dtype=torch.uint8, device=dev)
                dq = torch.full((T, Hq, d), float("nan"), device=dev)
                dk = torch.full((T, Hkv, d), float("nan"), device=dev)
                dv = torch.full((T, Hkv, d), float("nan"), device=dev)
                st = _lib.bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), ob.data_ptr(),
                                  ob.data_ptr(), lz.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), B, Hq, Hkv, N, d, 1, scale, cu.data_ptr(),
                                  ws.data_ptr(), ws.numel(), st_, fa.FA_BF16, fa.FA_BF16,
                                  fa.FA_F32)
                torch.cuda.synchronize()
                assert st == S[want], (label, entry, st)
                assert torch.isnan(dq).all() and torch.isnan(dk).all(), (label, entry)
                continue
            torch.cuda.synchronize()
            assert st == S[want], (label, entry, st)
            if want == "FA_OK":
                assert torch.isfinite(o).all(), (label, entry)
            else:
                assert torch.isnan(o).all() and torch.isnan(lse).all(), (label, entry)
            print(f"  {entry}: status {st}", flush=True)
    # The predicate itself, on the host, agrees with the device outcomes.
    for label, offs, want in cases:
        assert fa.check_seqlens(np.array(offs, np.int32), len(offs) - 1, N) == S[want]
    print("DEBUG_SEQLENS_OK", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
