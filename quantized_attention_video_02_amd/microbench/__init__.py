"""Microbenchmarks of the MI355X units the attention kernels are bound by
(mb.hip): dense INT8 / FP8 / FP16 MFMA rates, v_exp_f32 rate, and the
device-to-device copy bandwidth.  Run: python -m quantized_attention_video_02_amd.microbench"""
