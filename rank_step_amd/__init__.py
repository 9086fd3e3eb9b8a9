"""rank_step_amd: one FSDP FULL_SHARD rank's optimizer step on MI355X (gfx950).

The work runs in the HIP library ``librank_step.so`` (sources in ``csrc/``);
``rank_step_amd.binding`` marshals arguments to its C-ABI and nothing else.
The library is loaded on first use; every entry point raises if it is missing.
"""
