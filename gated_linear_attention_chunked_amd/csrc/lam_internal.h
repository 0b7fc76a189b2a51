// lam_internal.h -- launch descriptors shared by the C ABI layer and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lam {

enum Variant { kDeltaNet = 0, kGatedDeltaNet = 1, kKimiDelta = 2, kGatedDeltaNet2 = 3 };
enum DType { kF32 = 0, kBF16 = 1 };

// Validated arguments of one delta-rule scan.  Pointers are device pointers;
// sizes are already checked for range and overflow.
struct DeltaArgs {
    int variant, dtype;
    int64_t B, T, H;
    int dk, dv;
    const void *q, *k, *v, *alpha, *erase_b, *write_w, *beta;
    const float *state_in;
    void *out;
    float *state_out;
};

struct VlaArgs {
    int dtype;
    int64_t B, T, H;
    int d;
    const void *q, *k, *v, *p;
    const float *A_in, *S_in;
    void *out;
    float *A_out, *S_out;
};

// Each launcher enqueues its kernels on `stream` and returns the HIP status of
// the launch.  The caller has validated every argument.
hipError_t launch_delta_recurrent(const DeltaArgs &a, hipStream_t stream);
hipError_t launch_vla_recurrent(const VlaArgs &a, hipStream_t stream);

// Chunked schedule: returns hipErrorNotSupported (without launching) when no
// chunked kernel is built for the variant / dtype / head sizes.
bool delta_chunked_supported(const DeltaArgs &a);
hipError_t launch_delta_chunked(const DeltaArgs &a, hipStream_t stream);
// VLA chunked schedule (fp32 matrix cores, any dtype of the token streams).
bool vla_chunked_supported(const VlaArgs &a);
hipError_t launch_vla_chunked(const VlaArgs &a, hipStream_t stream);

// Device workspace of `bytes` for the chunked schedules' derived blocks, kept
// per (device, stream) and grown on demand.  Work queued on `stream` may use
// it until the next call on that stream that asks for more.
hipError_t derived_workspace(hipStream_t stream, size_t bytes, void **ptr);

// Kimi Delta (per-channel decay) has its own chunked kernel.
bool kda_chunked_supported(const DeltaArgs &a);
hipError_t launch_kda_chunked(const DeltaArgs &a, hipStream_t stream);

}  // namespace lam
