// lam_internal.h -- launch descriptors shared by the C ABI layer and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
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
    // Caller-provided workspace (chunked schedules only): the status block
    // (kStatusBytes, word 0 = device error bits), then the derived blocks.
    void *ws;
    // Per-token routing signal [B,T,H,dv] in the storage dtype, or NULL:
    // the residual r (kSideResidual) or the write value (kSideValue).
    void *side;
    int side_kind;
};
enum { kSideNone = 0, kSideResidual = 1, kSideValue = 2 };

struct VlaArgs {
    int dtype;
    int64_t B, T, H;
    int d;
    const void *q, *k, *v, *p;
    const float *A_in, *S_in;
    void *out;
    float *A_out, *S_out;
    void *ws;
    // ratio read (token-recurrent kernel only): the denominator state [B,H,d]
    bool ratio;
    const float *n_in;
    float *n_out;
};

// Size of the status block at the start of every workspace; the derived
// blocks follow it, so they keep the workspace's 256-byte alignment.
constexpr size_t kStatusBytes = 256;

// Each launcher enqueues its kernels on `stream` and returns the HIP status of
// the launch.  The caller has validated every argument.
hipError_t launch_delta_recurrent(const DeltaArgs &a, hipStream_t stream);
hipError_t launch_vla_recurrent(const VlaArgs &a, hipStream_t stream);

// Chunked schedule: returns hipErrorNotSupported (without launching) when no
// chunked kernel is built for the variant / dtype / head sizes.
bool delta_chunked_supported(const DeltaArgs &a);
// Workspace bytes of the chunked schedule for a.B, a.T, a.H, a.dk, a.dv
// (status block included); false when the call has more chunk tasks than
// one grid takes.
bool delta_chunked_workspace(const DeltaArgs &a, size_t *bytes);
// Enqueues the chunked kernels; a.ws holds at least
// delta_chunked_workspace(a) bytes.
hipError_t launch_delta_chunked(const DeltaArgs &a, hipStream_t stream);
// The fp32 chunked form of DeltaNet, Gated DeltaNet and Gated DeltaNet-2
// (16-token chunks on fp32 matrix cores, any storage dtype, dk in {32, 64,
// 96, 128}, dv a multiple of 16): the chunked schedule for the shapes the
// bf16 one does not take.  Workspace: the status block, then one chunk record
// per (b, h, 16-token chunk).
bool delta_f32_chunked_supported(const DeltaArgs &a);
bool delta_f32_chunked_workspace(const DeltaArgs &a, size_t *bytes);
hipError_t launch_delta_f32_chunked(const DeltaArgs &a, hipStream_t stream);
// VLA chunked schedule (fp32 matrix cores, any dtype of the token streams).
bool vla_chunked_supported(const VlaArgs &a);
bool vla_chunked_workspace(const VlaArgs &a, size_t *bytes);
hipError_t launch_vla_chunked(const VlaArgs &a, hipStream_t stream);

// One-token decode step, memory updated in place (state_in == state_out).
bool delta_step_supported(const DeltaArgs &a);
hipError_t launch_delta_step(const DeltaArgs &a, hipStream_t stream);

// Backward pass: the forward's inputs in f (out, state_out unused; ws = the
// workspace), the output and final-state adjoints, and fp32 gradients.
struct DeltaBwdArgs {
    DeltaArgs f;
    const void *dout;          // [B,T,H,dv], storage dtype
    const float *dstate_out;   // [B,H,dv,dk] or NULL
    float *dq, *dk, *dv, *dalpha, *derase_b, *dwrite_w, *dbeta, *dstate_in;
    float *ckpt;               // states every 16 tokens, [B*H][chunks][dv][dk]
};
bool delta_backward_workspace(const DeltaArgs &a, size_t *bytes);
hipError_t launch_delta_backward(const DeltaBwdArgs &g, hipStream_t stream);
// The chunked backward of DeltaNet, Gated DeltaNet and Gated DeltaNet-2 on
// fp32 matrix cores (shapes as delta_f32_chunked_supported, T > 0): the
// derivation with the adjoint records, the forward again keeping each
// chunk's start state and residuals, the adjoint scan in reverse, and the
// chunk-parallel gradients.  Workspace: the status block, the records, the
// per-chunk states and state cotangents, U and dX.
bool delta_f32_backward_workspace(const DeltaArgs &a, size_t *bytes);
hipError_t launch_delta_f32_backward(const DeltaBwdArgs &g, hipStream_t stream);

// Log-linear (Fenwick-tree) readout: f as the plain scan (state_in /
// state_out are level states [B,H,nL,dv,dk]), nL levels, t0 = absolute
// position of token 0, lam = level weights [B,T,H,nL] fp32.
constexpr int kLogLinMaxLevels = 24;   // positions below 2^23
constexpr int kLogLinMaxHidden = 64;   // hidden width of the level-weight MLP
struct LogLinArgs {
    DeltaArgs f;
    int nL;
    int64_t t0;
    const float *lam;
};
bool loglin_supported(const DeltaArgs &a, int nL);
hipError_t launch_loglin(const LogLinArgs &g, hipStream_t stream);
hipError_t launch_loglin_lambda(int dtype, int64_t M, int nL, int nh, const void *d, const float *W1,
                                const float *W2, const float *b, float *lam, hipStream_t stream);

// Routing epilogue h += s P^T (s [M,N], P [D,N], h [M,D], one dtype).
bool route_supported(int64_t D, int64_t N);
hipError_t launch_route(int dtype, int64_t M, int64_t D, int64_t N, const void *s, const void *P, void *h,
                        hipStream_t stream);

// Kimi Delta (per-channel decay) has its own chunked kernel.
bool kda_chunked_supported(const DeltaArgs &a);
bool kda_chunked_workspace(const DeltaArgs &a, size_t *bytes);
hipError_t launch_kda_chunked(const DeltaArgs &a, hipStream_t stream);

}  // namespace lam
