"""The roofline denominators bench.py reports: algorithmic bytes (every input
read once, y and the final state written once, at the storage width) and
algorithmic flops (7 dk dv per token-head for the delta rule, 12 d^2 for
VLA), checked against counts worked out by hand from each workload's shapes.
CPU only."""
import bench
from gated_linear_attention_chunked_amd import inputs as I

# (bytes, flops) per workload, from its shapes:
#   bytes = B*T*H * (per-token-head bytes) + final state(s) in fp32
#   flops = B*T*H * 7*dk*dv (delta rule) or 12*d^2 (VLA)
EXPECTED = {
    # fp32: q, k, v, out 4 x 32 x 4 B + beta 4 B = 516 B x 512 token-heads, + 1x2x32x32x4 B state
    "deltanet_f32_B1_T256_H2_d32": (516 * 512 + 8192, 7 * 32 * 32 * 512),
    # bf16: q, k, v, out 4 x 128 x 2 B + alpha 2 + beta 2 = 1028 B x 262,144, + 8x8x128x128x4 B
    "gdn_bf16_B8_T4096_H8_d128": (273_678_336, 30_064_771_072),
    # bf16: 1028 + per-channel alpha 256 - scalar alpha 2 = 1282 B x 524,288, + 2x8x128x128x4 B
    "kda_bf16_B2_T32768_H8_d128": (673_185_792, 60_129_542_144),
    # bf16: 1028 + erase 256 + write 256 = 1540 B x 262,144, + state
    "gdn2_bf16_B8_T4096_H8_d128": (407_896_064, 30_064_771_072),
    # fp32: q, k, v, p, out 5 x 32 x 4 B = 640 B x 131,072, + A and S 2 x 4x8x32x32x4 B
    "vla_f32_B4_T4096_H8_d32": (84_148_224, 12 * 32 * 32 * 131_072),
    # fp32: 5 x 96 x 4 = 1920 B x 131,072, + 2 x 4x8x96x96x4 B
    "vla_f32_B4_T4096_H8_d96": (254_017_536, 12 * 96 * 96 * 131_072),
}


def test_every_workload_is_counted():
    assert set(EXPECTED) == set(I.WORKLOADS)


def test_algorithmic_bytes_and_flops():
    for name, (nbytes, nflops) in EXPECTED.items():
        w = I.WORKLOADS[name]
        assert bench.algorithmic_bytes(w) == nbytes, name
        assert bench.algorithmic_flops(w) == nflops, name


def test_metric_workload_is_hbm_bound_at_peak():
    """At the published peaks the Gated DeltaNet workload's bytes take longer
    than its flops on bf16 matrix cores (34.2 us vs 12.0 us), so its
    roofline is HBM."""
    w = I.WORKLOADS[I.METRIC_WORKLOAD]
    t_hbm = bench.algorithmic_bytes(w) / (bench.HBM_PEAK_GBS * 1e9)
    t_mfma = bench.algorithmic_flops(w) / (bench.MFMA_BF16_PEAK_TFS * 1e12)
    assert abs(t_hbm - 34.2e-6) < 0.1e-6 and t_mfma < t_hbm


# (bytes, flops) per call of the jobs beside the forward scan, worked out by
# hand for B8 T4096 H8 dk = dv = 128, bf16 streams (262,144 token-heads):
JOB_EXPECTED = {
    # reads q, k, v, dout 4 x 128 x 2 + beta 2 + alpha 2 = 1028 B; writes dq, dk, dv
    # 3 x 128 x 4 + dbeta 4 + dalpha 4 = 1544 B; + dstate_in 4,194,304 B.
    # flops 14 x 128 x 128 per token-head
    "gdn_bwd_bf16_B8_T4096_H8_d128": (2572 * 262_144 + 4_194_304, 14 * 16_384 * 262_144),
    # the forward's 273,678,336 B + the residual 128 x 2 B per token-head
    "gdn_side_bf16_B8_T4096_H8_d128": (273_678_336 + 256 * 262_144, 7 * 16_384 * 262_144),
    # M = 32,768 tokens, N = 1024, D = 1024: (M N + D N + 2 M D) x 2 B; 2 M N D flops
    "route_bf16_B8_T4096_N1024_D1024": (203_423_744, 68_719_476_736),
    # 13 levels: forward bytes - one state + lambda 13 x 4 B per token-head + 13 states;
    # occupancy sum over t < 4096 of popcount(t) + 1 = 4096 x 6 + 4096 = 28,672
    "gdn_loglinear_bf16_B8_T4096_H8_d128": (273_678_336 - 4_194_304 + 52 * 262_144 + 13 * 4_194_304,
                                            64 * 28_672 * 7 * 16_384),
    # d (13 x 2 B) in, lambda (13 x 4 B) out per row; 4 x 13 x 26 flops per row
    "loglinear_lambda_bf16_B8_T4096_H8_L13": (78 * 262_144, 1352 * 262_144),
}


def test_job_counts():
    forward_jobs = {n for n, j in bench.JOBS.items() if j[0] == "forward"}
    assert set(JOB_EXPECTED) == set(bench.JOBS) - forward_jobs
    # the fp32-storage forward job is a plain forward: q, k, v, out (4 x 8 x 4096
    # x 8 x 128 x 4 B), alpha and beta (2 x 8 x 4096 x 8 x 4 B), the final
    # state (64 x 128 x 128 x 4 B)
    kind, base, extra = bench.JOBS["gdn_f32_B8_T4096_H8_d128"]
    w = I.WORKLOADS[base].replace(dtype=extra["dtype"])
    assert bench.algorithmic_bytes(w) == 4 * 134_217_728 + 2 * 1_048_576 + 4_194_304
    for name, (nbytes, nflops) in JOB_EXPECTED.items():
        kind, base, extra = bench.JOBS[name]
        assert bench.job_counts(kind, I.WORKLOADS[base], extra) == (nbytes, nflops), name


def test_loglinear_levels_and_occupancy():
    assert [bench.loglinear_levels(T) for T in (1, 2, 3, 4, 5, 4096, 4097)] == [1, 2, 3, 3, 4, 13, 14]
    # positions 0..7: popcounts 0,1,1,2,1,2,2,3 -> 12, plus one level 0 each -> 20
    assert bench.loglinear_occupancy(8) == 20


def test_decode_counts():
    """Decode steps read and write the state they update.  Gated DeltaNet
    N256 H8 d128 bf16: 1028 B per stream-head (q, k, v, out, alpha, beta) +
    the fp32 state read and written (2 x 65,536 B).  VLA with the ratio read,
    N256 H8 d96 fp32: q, k, v, p, out 5 x 96 x 4 = 1920 B, A and S read and
    written 4 x 96 x 96 x 4 = 147,456 B, the denominator read and written
    2 x 96 x 4 = 768 B, per stream-head."""
    g = I.DECODE_WORKLOADS["gdn_step_bf16_N256_H8_d128"]
    assert bench.algorithmic_bytes(g, True) == 2048 * 1028 + 2 * 2048 * 65_536
    v = I.DECODE_WORKLOADS["vla_ratio_step_f32_N256_H8_d96"]
    assert bench.algorithmic_bytes(v, True) == 2048 * (1920 + 147_456 + 768)
    assert bench.algorithmic_flops(v) == 2048 * 12 * 96 * 96
