"""Device buffers of one attention layer's paged KV cache and its selection
state, with the three library calls bound to them.

torch only allocates device memory and supplies the stream; every step of the
computation runs in libnsa's kernels.
"""

from __future__ import annotations

import torch

from . import _abi as A

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}
_NSA_DTYPE = {"bf16": A.NSA_BF16, "f32": A.NSA_F32}
_MODE = {"group_softmax": A.NSA_SCORE_GROUP_SOFTMAX, "forecast": A.NSA_SCORE_FORECAST_RAW,
         "forecast_window": A.NSA_SCORE_FORECAST_WINDOW}


class SparseDecodeLayer:
    """One layer: pools [P][Hkv][64][D], block table, reps, eviction state.

    Attributes are plain torch tensors; fill ``k_pool``, ``v_pool``,
    ``block_table``, ``evict_logits`` and ``seq_lens`` directly.
    """

    def __init__(self, *, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 max_blocks_per_seq: int, num_phys_blocks: int, dtype: str = "bf16",
                 mode: str = "group_softmax", k: int = 64, k_e: int = 0,
                 ordered: bool = False, tau: float = 0.0, softmax_scale: float = 0.0,
                 device="cuda", eviction_logits: bool = True):
        self.B, self.Hq, self.Hkv, self.D = batch, num_q_heads, num_kv_heads, head_dim
        self.G = num_q_heads // num_kv_heads
        self.max_blocks, self.P = max_blocks_per_seq, num_phys_blocks
        self.dtype, self.mode = dtype, mode
        self.k, self.k_e, self.ordered, self.tau = k, k_e, ordered, tau
        self.device = torch.device(device)
        self.shape = A.Shape.make(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                  num_phys_blocks, _NSA_DTYPE[dtype], softmax_scale)
        self.sel_params = A.SelectParams(_MODE[mode], k, 0 if ordered else k_e, int(ordered))
        self.dec_params = A.DecodeParams(k, int(ordered), float(tau))
        td, dev = _TORCH_DTYPE[dtype], self.device
        B, H, D, MB = batch, num_kv_heads, head_dim, max_blocks_per_seq
        self.k_pool = torch.zeros((num_phys_blocks, H, 64, D), dtype=td, device=dev)
        self.v_pool = torch.zeros((num_phys_blocks, H, 64, D), dtype=td, device=dev)
        self.block_table = torch.zeros((B, MB), dtype=torch.int32, device=dev)
        self.seq_lens = torch.zeros(B, dtype=torch.int32, device=dev)
        self.evict_logits = (torch.zeros((B, H, MB * 64), dtype=torch.float32, device=dev)
                             if eviction_logits else None)
        self.reps = torch.zeros((B, H, MB, 4, D), dtype=td, device=dev)
        self.evict_scores = (torch.zeros((B, H, MB), dtype=torch.float32, device=dev)
                             if eviction_logits else None)
        self.evict_set = torch.full((B, H, max(k_e, 1)), -1, dtype=torch.int32, device=dev)
        self.evict_seen = torch.zeros((B, H), dtype=torch.int32, device=dev)
        self.selected = torch.full((B, H, k), -1, dtype=torch.int32, device=dev)
        self.num_selected = torch.zeros((B, H), dtype=torch.int32, device=dev)
        self.num_processed = torch.zeros((B, H), dtype=torch.int32, device=dev)
        self.out = torch.zeros((B, num_q_heads, D), dtype=td, device=dev)
        cap = 64 * MB
        self.sel_ws_bytes = A.nsa_select_workspace_bytes(self.shape, self.sel_params, cap)
        self.dec_ws_bytes = A.nsa_decode_workspace_bytes(self.shape, self.dec_params)
        self.sel_ws = torch.zeros(self.sel_ws_bytes, dtype=torch.uint8, device=dev)
        self.dec_ws = torch.zeros(self.dec_ws_bytes, dtype=torch.uint8, device=dev)
        # the fused step's workspace (ascending mode only), zeroed once here:
        # every completed step leaves its hand-off slots zero again
        self.step_ws, self.step_ws_bytes = None, 0
        if not ordered:
            try:
                self.step_ws_bytes = A.nsa_decode_step_workspace_bytes(self.shape, self.sel_params,
                                                                       cap)
            except A.NsaError as e:
                if e.status != A.NSA_ERR_UNSUPPORTED:
                    raise
            else:
                self.step_ws = torch.zeros(self.step_ws_bytes, dtype=torch.uint8, device=dev)

    # -- the three calls ---------------------------------------------------
    def update_reps(self, first_block: torch.Tensor, num_blocks: torch.Tensor,
                    max_num_blocks: int, stream=None) -> None:
        A.nsa_update_block_reps(self.shape, self.k_pool, self.block_table, self.evict_logits,
                                first_block, num_blocks, max_num_blocks, self.reps,
                                self.evict_scores, stream)

    def select(self, query: torch.Tensor, max_seq_len: int, stream=None) -> None:
        ke = self.k_e > 0 and not self.ordered
        A.nsa_select_blocks(self.shape, self.sel_params, query, self.reps,
                            self.evict_scores if ke else None, self.seq_lens, max_seq_len,
                            self.evict_set if ke else None, self.evict_seen if ke else None,
                            self.selected, self.num_selected, self.sel_ws, self.sel_ws_bytes,
                            stream)

    def decode(self, q: torch.Tensor, stream=None, selected=None, num_selected=None,
               max_selected=None, early_stop=None, bias=None) -> None:
        """Attention over the selected blocks and the tail.  bias: None, or
        the per-token additive logits [B][Hkv][64 * max_blocks] float32
        (the eviction logits, ED-DMA variant: nsa_sparse_decode_biased)."""
        params = self.dec_params
        if max_selected is not None or early_stop is not None:
            params = A.DecodeParams(max_selected or self.k,
                                    int(self.ordered if early_stop is None else early_stop),
                                    float(self.tau))
            need = A.nsa_decode_workspace_bytes(self.shape, params)
            if need > self.dec_ws_bytes:
                self.dec_ws = torch.zeros(need, dtype=torch.uint8, device=self.device)
                self.dec_ws_bytes = need
        sel = self.selected if selected is None else selected
        nsel = self.num_selected if num_selected is None else num_selected
        if bias is not None:
            A.nsa_sparse_decode_biased(self.shape, params, q, self.k_pool, self.v_pool,
                                       self.block_table, self.seq_lens, sel, nsel, bias,
                                       self.num_processed, self.out, self.dec_ws,
                                       self.dec_ws_bytes, stream)
            return
        A.nsa_sparse_decode(self.shape, params, q, self.k_pool, self.v_pool, self.block_table,
                            self.seq_lens, sel, nsel, self.num_processed, self.out, self.dec_ws,
                            self.dec_ws_bytes, stream)

    def step(self, query: torch.Tensor, q: torch.Tensor, max_seq_len: int, stream=None) -> None:
        """Selection and decode in one launch (ascending mode).  Enqueues only:
        call check_step() where the results are consumed."""
        if self.step_ws is None:
            raise A.NsaError(A.NSA_ERR_UNSUPPORTED,
                             "nsa_decode_step: not available for this layer (ordered mode, or "
                             "a context above the fused step's limit)")
        ke = self.k_e > 0
        A.nsa_decode_step(self.shape, self.sel_params, query, q, self.reps,
                          self.evict_scores if ke else None, self.k_pool, self.v_pool,
                          self.block_table, self.seq_lens, max_seq_len,
                          self.evict_set if ke else None, self.evict_seen if ke else None,
                          self.selected, self.num_selected, self.out, self.step_ws,
                          self.step_ws_bytes, stream)

    def step_noalloc(self, query: torch.Tensor, q: torch.Tensor, max_seq_len: int,
                     step_status=None, stream=None) -> None:
        """The fused step on the library's own per-device workspace (no
        workspace argument).  step_status: None or a one-element int32 device
        tensor, set to 1 if a wait of the step expired."""
        ke = self.k_e > 0
        A.nsa_decode_step_noalloc(self.shape, self.sel_params, query, q, self.reps,
                                  self.evict_scores if ke else None, self.k_pool, self.v_pool,
                                  self.block_table, self.seq_lens, max_seq_len,
                                  self.evict_set if ke else None,
                                  self.evict_seen if ke else None, self.selected,
                                  self.num_selected, self.out, step_status, stream)

    def residency_diff(self, prev_selected, prev_num_selected, prev_seq_lens, fetch, num_fetch,
                       release, num_release, gamma=None, stream=None) -> None:
        """Blocks to fetch and to release from the previous selection (given)
        to the current one (this layer's selected / num_selected)."""
        A.nsa_residency_diff(self.shape, self.k, prev_selected, prev_num_selected, prev_seq_lens,
                             self.selected, self.num_selected, fetch, num_fetch, release,
                             num_release, gamma, stream)

    def check_step(self, stream=None) -> None:
        """Raise NsaError(NSA_ERR_STEP_EXPIRED) if a wait of a fused step on
        this layer expired since the last check (synchronises the stream; the
        workspace is cleared, and the eviction state is the one before the
        failed step, so the step can be run again)."""
        if self.step_ws is not None:
            A.nsa_decode_step_status(self.step_ws, self.step_ws_bytes, True, stream)

    def reset_state(self) -> None:
        self.evict_set.fill_(-1)
        self.evict_seen.zero_()
