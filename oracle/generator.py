"""Oracle for one generator frame: the delayed-code ring, the temporal step, text
sampling and the sampled depth loop (fp64, NumPy, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring. Never called by the library.

Source: "PersonaPlex native LM audit" (Clockless Inkling, personaplex-research page),
"Generator delayed-code cache" and section 7 "One exact generator step": a ring of 17
streams x 4 slots of integer codes with a "provided" flag per entry, a cursor s, and per
stream delays text 0, agent codebook 0 delay 0, agent codebooks 1-7 delay 1, user
codebook 0 delay 0, user codebooks 1-7 delay 1 (maximum delay 1). One call at cursor s:

  1. supplied codes (user audio; optionally agent text or codes) go to slot
     (s + delay_k) mod 4 of their stream, marked provided;
  2. at s = 0 the first slot receives the initial tokens (text 32000, audio 2048) -- here
     wherever that entry was not supplied -- the cursor advances and there is no output;
  3. the temporal input is slot (s - 1) mod 4, the target slice slot s mod 4;
  4. temporal step, text logits, text sample -- a supplied text target replaces it for
     the depth conditioning;
  5. depth positions 0..15 (streams 1..16): sample, or take the supplied target where
     provided; the selected code feeds the next position;
  6. the selections are written into the target slots that were not supplied; the
     consumed input slot's provided flags are cleared;
  7. once the initial delay padding is over (s >= 2), the aligned output of stream k is
     slot (s - 1 + delay_k) mod 4; the cursor advances.

Readings (the page leaves them open): random draws are inputs (one uniform for the text
sample and one per depth position, 17 per frame); the initial tokens do not overwrite a
supplied entry of the first slot; the temporal position counts model steps from 0 (the
first model step is at cursor 1).
"""

import numpy as np

from . import depformer as OD
from . import temporal as O
from .sampling import sample_top_k

N_STREAMS = 17
RING = 4
DELAYS = (0, 0, 1, 1, 1, 1, 1, 1, 1, 0, 1, 1, 1, 1, 1, 1, 1)
MAX_DELAY = 1
TEXT_INITIAL = 32000
AUDIO_INITIAL = 2048


class Generator:
    """Generator state for one session: the code ring, its provided flags, the cursor and
    the temporal KV history (the depth history is per frame)."""

    def __init__(self, W_t, cfg_t, W_d, cfg_d, text_temperature=0.7, text_top_k=25,
                 audio_temperature=0.8, audio_top_k=250):
        self.W_t, self.cfg_t, self.W_d, self.cfg_d = W_t, cfg_t, W_d, cfg_d
        self.tt, self.tk = text_temperature, text_top_k
        self.at, self.ak = audio_temperature, audio_top_k
        self.tok = np.full((N_STREAMS, RING), -1, np.int64)
        self.prov = np.zeros((N_STREAMS, RING), bool)
        self.s = 0
        self.pos = 0
        self.cache = O.Cache(cfg_t["n_layers"])
        self.last_inputs = None          # temporal input IDs of the last model step
        self.last_chosen = None          # the 17 selections of the last model step
        self.last_h = None               # its final-normed temporal hidden
        self.last_text_logits = None     # and its text logits
        self.last_depth_logits = None    # [n_steps, n_out] depth logits of the last model step

    def step(self, provided=None, uniforms=None):
        """One call. provided: length-17 codes (-1 = not supplied); user audio is streams
        9..16. uniforms: 17 draws in [0, 1) (text, then depth positions 0..15).
        Returns the aligned 17 output codes, or None while the initial padding lasts."""
        s = self.s
        if provided is not None:
            for k in range(N_STREAMS):
                if int(provided[k]) >= 0:
                    slot = (s + DELAYS[k]) % RING
                    self.tok[k, slot] = int(provided[k])
                    self.prov[k, slot] = True
        if s == 0:
            for k in range(N_STREAMS):
                if not self.prov[k, 0]:
                    self.tok[k, 0] = TEXT_INITIAL if k == 0 else AUDIO_INITIAL
            self.s = 1
            return None
        src, tgt = (s - 1) % RING, s % RING
        ids = self.tok[:, src].copy()
        self.last_inputs = ids
        x = O.decode_step(O.embed(ids, self.W_t, self.cfg_t), self.pos, self.cache, self.W_t, self.cfg_t)
        self.pos += 1
        h, text_logits = O.final(x, self.W_t, self.cfg_t, with_logits=True)
        self.last_h = h
        self.last_text_logits = text_logits
        u = np.zeros(N_STREAMS) if uniforms is None else np.asarray(uniforms, np.float64)
        text = sample_top_k(text_logits, self.tt, self.tk, u[0])
        if self.prov[0, tgt]:
            text = int(self.tok[0, tgt])

        def select(q, lg):
            k = q + 1
            if self.prov[k, tgt]:
                return int(self.tok[k, tgt])
            return sample_top_k(lg, self.at, self.ak, u[k])

        codes, self.last_depth_logits = OD.step_select(h, text, select, self.W_d, self.cfg_d)
        chosen = [text] + [int(c) for c in codes]
        self.last_chosen = np.array(chosen, np.int64)
        for k in range(N_STREAMS):
            if not self.prov[k, tgt]:
                self.tok[k, tgt] = chosen[k]
        self.prov[:, src] = False
        out = None
        if s >= MAX_DELAY + 1:
            out = np.array([self.tok[k, (s - MAX_DELAY + DELAYS[k]) % RING] for k in range(N_STREAMS)], np.int64)
        self.s = s + 1
        return out
