"""MI355X-native hot path of Introspective Strided Decoding (ISD).

`strided_verify_propose_amd.isd` binds the HIP library (attention_step, verify,
gated_lora_proj); `strided_verify_propose_amd.synth` builds seeded synthetic inputs.
Importing the package loads nothing: the library is opened on first use.
"""
