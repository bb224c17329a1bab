"""ReplaySSM decode step for MI355X (gfx950): checkpoint + input ring, replay outputs, flush,
speculative append/rollback and a low-precision read copy, behind a C ABI (include/ssm_replay.h).

    from ssm_decode_state_amd import binding   # loads libssm_replay.so (fails loudly if unbuilt)
    from ssm_decode_state_amd import synth     # seeded synthetic inputs
"""
