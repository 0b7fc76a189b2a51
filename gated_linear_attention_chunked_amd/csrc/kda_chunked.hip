// kda_chunked.hip -- chunked Kimi Delta scan (per-channel decay) on gfx950
// matrix cores; bf16 streams, fp32 state.
//
// The rule ("Mechanisms, trade-offs and cross-layer routing of
// linear-attention architectures", "Technical details"): Kimi Delta decays the
// memory channel by channel along the key-feature axis, W~ = W diag(a_t), and
// writes the residual of W~ k_t along k_t: W_t = W~ + beta_t (v_t - W~ k_t) k_t^T,
// y_t = W_t q_t.
//
// Chunked form over C = 16 tokens (rows = tokens, S = memory at the chunk
// start, G_t = sum_{j<=t} log2 a_j per channel, Gam_t = 2^{G_t}):
//   N   = strict_lower((K * Gam) (K / Gam)^T)
//   R   = (I + N diag(beta))^{-1} (V - (K * Gam) S^T)
//   Y   = (Q * Gam) S^T + lower((Q * Gam) (K / Gam)^T) diag(beta) R
//   S'  = S diag(Gam_C) + R^T diag(beta) (K * Gam_C / Gam)
// Row t of R is token t's residual against the decayed memory (the write is
// beta_t r_t k_t^T); beta is folded into the derived tiles that consume R,
// so the scan carries the residual itself.
// Every entry of the two Gram-type products is sum_c x_tc k_sc 2^{G_tc - G_sc}
// with s <= t, at most |x_t||k_s|.  Splitting 2^{G_t - G_s} into 2^{G_t} and
// 2^{-G_s} puts both products on MFMA; 2^{-G_s} stays finite while the decay
// over the chunk keeps every channel above 2^-100.  A chunk that decays
// further (alpha near zero somewhere) takes an exact path instead: each entry
// is summed channel by channel with 2^{G_tc - G_sc} <= 1 evaluated directly.
// C = 16 makes the Gram a single 16x16 block, so one factorisation serves the
// whole sub-chunk.
//
// The scan steps over pairs of 16-token sub-chunks (32 tokens).  Both
// sub-chunks act on the state at the pair start: the odd one's K * Gam and
// Q * Gam carry the even one's decay, the even one's K * Gam_C / Gam the odd
// one's, and the coupling between them is a 16x16 block per product,
//   G_10 = (K_1 * Gam_1)(K_0 * Gam_C0 / Gam_0)^T,  Aqk_10 = (Q_1 * Gam_1)(K_0 * Gam_C0 / Gam_0)^T,
// whose factors split at the last even token and are both at most 1, so
// they need no exact form.  Then R_0 = D_0 (V_0 - Z_0),
// R_1 = D_1 (V_1 - Z_1) + M_10 R_0 with M_10 = -D_1 G_10 diag(beta_0) and
// D_i = (I + N_ii diag(beta_i))^{-1}, and one 32-token state update: one
// more dependent product than a 16-token step, for half as many steps.
//
// Two kernels per call:
//   derivation: one wave per (sequence, head, sub-chunk), all sub-chunks at
//          once (a wholly padded odd sub-chunk completes the last pair).  It
//          forms everything that does not depend on the state: the scaled
//          key and query tiles, the Aqk block, (I + L)^{-1} diag(beta), the
//          pair's Gam_C and (odd sub-chunks) M_10 and Aqk_10, and writes them
//          to a workspace block per sub-chunk.
//   scan:  one workgroup per (b, h, value slice of 16 NVT columns):
//   carry  (NVT waves, one 16-column tile each): Z = (K*Gam) S^T for both
//          sub-chunks, the two 16x16 solves and the coupling on three MFMA,
//          state update S^T <- diag(Gam_C) S^T + (beta K*Gam_C/Gam)^T R over the
//          32 tokens, bf16 copy of S published for the output.
//   output (NVT waves): from the published bf16 S it forms R exactly as the
//          carry does (same operands, same order), then Y^T = S (Q*Gam)^T +
//          R^T Aqk^T, 8-byte row stores.  Recomputing R costs the output a
//          few products and takes a hand-off off the carry's chain.
//   producers (4 waves): producer p copies every fourth pair's two blocks
//          (p, p+4, ...) and the slice's value rows into its own LDS slot,
//          loads issued four pairs ahead.
// There is no workgroup barrier in the chunk loop: slots, R and the bf16
// state move between roles through bounded LDS counters.
#include <type_traits>

#include "chunk_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

constexpr int C16 = 16;      // chunk length (tokens)
constexpr int NSLOT = 4;     // one chunk slot per producer
constexpr int KLTS = 20;     // column stride (floats) of the fp32 L block
constexpr float kFastLimit = 100.f;  // largest 2^x used by the factored Gram

// NVT 16-column value tiles per workgroup: one carry and one output wave
// each, plus four producers.
template <int NVT>
struct KdaShape {
    static constexpr int BV = 16 * NVT;       // dv columns per workgroup
    static constexpr int NW = 2 * NVT + 4;    // waves
    static constexpr int NT = 64 * NW;        // threads
};

// State-independent data of one chunk as the derivation kernel stores it:
// token rows unpadded, fragments in the order the scan reads them.
template <int DK>
struct KdaBlock {
    __bf16 kd[C16 * DK];   // k * Gam
    __bf16 ke[C16 * DK];   // beta k * Gam_C / Gam
    __bf16 qd[C16 * DK];   // q * Gam
    bf16x4 aqk[64];        // lower((Q*Gam)(K/Gam)^T) diag(beta), B-operand order: lane (g, i) holds [t = i][s = 4g + r]
    bf16x4 dt[64];         // D = (I + N diag(beta))^{-1}, A-operand order
    float gc[DK];          // even sub-chunk: Gam_C of the pair, per channel
    bf16x4 mx[64];         // odd sub-chunk: M_10 = -D_1 G_10 diag(beta_0), A-operand order
    bf16x4 ax[64];         // odd sub-chunk: cross block of Aqk (times beta_0), B-operand order: lane (g, i) holds [t = i][s = 4g + r]
    static constexpr int kRowPieces = 3 * C16 * DK / 8;            // 16-byte pieces of kd, ke, qd
    static constexpr int kPieces = kRowPieces + 64 + DK / 4 + 64;  // all 16-byte pieces
};
static_assert(sizeof(KdaBlock<64>) % 256 == 0 && sizeof(KdaBlock<128>) % 256 == 0, "blocks stay 256-byte aligned");

template <int DK, int NVT>
struct KdaLds {
    static constexpr int KS = DK + 8;
    static constexpr int VS = KdaShape<NVT>::BV + 8;
    struct Slot {  // one pair of sub-chunks: their blocks (token rows padded to KS) and value rows
        alignas(16) __bf16 kd[2 * C16 * KS];   // rows 0-15 even sub-chunk, 16-31 odd
        alignas(16) __bf16 ke[2 * C16 * KS];
        alignas(16) __bf16 qd[2 * C16 * KS];
        alignas(16) bf16x4 aqk[2][64];
        alignas(16) bf16x4 dt[2][64];
        alignas(16) float gc[DK];              // Gam_C of the pair
        alignas(16) bf16x4 mx[64];
        alignas(16) bf16x4 ax[64];
        alignas(16) __bf16 v[2 * C16 * VS];    // value targets of the workgroup's columns
    };
    Slot slot[NSLOT];
    // A producer publishes chunk c only after every consumer has finished
    // chunk c - 4, so the carry can run at most four chunks ahead of the
    // output: with five state buffers the bf16 state needs no further check
    // (two when LDS is short, guarded by the output's read count).
    static constexpr int NSB = NVT == 1 ? 5 : 2;
    static constexpr bool kStateGuard = NSB < 5;
    alignas(16) bf16x4 sh[NSB][NVT][DK / 16][64];  // bf16 state per chunk and tile
    unsigned int ready[NSLOT];   // chunks published per slot
    unsigned int cons[NVT];      // chunks finished per output wave
    unsigned int sp[NVT], so[NVT];   // bf16 state published / read per tile
};

// ============================== derivation ==============================
template <int DK>
struct KdaDeriveLds {
    static constexpr int KS = DK + 8;
    alignas(16) __bf16 a[C16 * KS];    // k * Gam (factored form); row tiles of k (exact form)
    alignas(16) __bf16 b[C16 * KS];    // q * Gam (factored form); row tiles of q (exact form)
    alignas(16) __bf16 kb[C16 * KS];   // k / Gam (factored form); column tile (exact form)
    alignas(16) __bf16 k0[C16 * KS];   // odd sub-chunk: the even one's k * Gam_C / Gam (cross blocks)
    alignas(16) float lt[16 * KLTS];   // L by column
    alignas(16) float beta[C16];
    alignas(16) bf16x4 dt[64];
};

// One wave per (sequence, head, pair of 16-token sub-chunks), the even
// sub-chunk first.  Lane owns key channels CH*lane .. CH*lane + CH - 1 for all
// 16 tokens of a sub-chunk (one packed load per token and tensor); beta of
// token lane (lanes 0-15).
template <int DK>
__global__ __launch_bounds__(64) void kda_derive_kernel(DeltaArgs a, KdaBlock<DK> *__restrict__ out, int64_t Ts,
                                                        int64_t tb, unsigned int *status) {
    constexpr int KS = DK + 8;
    constexpr int KSTEP = DK / 32, CH = DK / 64;
    __shared__ KdaDeriveLds<DK> s;

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H);
    const int npair = (T + 2 * C16 - 1) / (2 * C16);  // pairs per head (the last may end in padding)
    const int task = blockIdx.x;
    const int head = task / npair, pr = task - head * npair;
    const int b = head / H, h = head % H;
    const int lane = threadIdx.x;
    const int lg = lane >> 4, lc = lane & 15;
    if (task == 0 && lane == 0) *status = 0u;  // first kernel of the call

    const uint16_t *gq = static_cast<const uint16_t *>(a.q);
    const uint16_t *gk = static_cast<const uint16_t *>(a.k);
    const uint16_t *gal = static_cast<const uint16_t *>(a.alpha);
    const uint16_t *gbe = static_cast<const uint16_t *>(a.beta);
    using Pk = std::conditional_t<CH == 2, uint32_t, uint16_t>;
    const int64_t hb = (static_cast<int64_t>(b) * Ts + tb) * H + h;  // token index of (b, tb, h)
    // rows are read clamped into the sequence (the odd sub-chunk may lie
    // wholly past its end) and padded: zero key and query, decay 1
    auto row = [&](int t) { return (hb + static_cast<int64_t>(min(t, T - 1)) * H) * DK + CH * lane; };
    const Pk one = CH == 2 ? Pk(0x3f803f80u) : Pk(0x3f80u);
    float gprev[CH];  // log2 Gam_C of the even sub-chunk, kept for the odd one
#pragma unroll 1
    for (int sub = 0; sub < 2; ++sub) {
        const int n = 2 * pr + sub;
        const bool odd = sub != 0;
        KdaBlock<DK> &o = out[2 * task + sub];
        wave_lds_fence();  // the previous sub-chunk's LDS reads before this one's writes
        Pk rk[C16], rq[C16], ra[C16];
        const int t0 = n * C16, nval = T - t0;  // nval <= 0: all padding
#pragma unroll
        for (int t = 0; t < C16; ++t) {
            const int64_t off = row(t0 + t);
            rk[t] = t < nval ? *reinterpret_cast<const Pk *>(gk + off) : Pk(0);
            rq[t] = t < nval ? *reinterpret_cast<const Pk *>(gq + off) : Pk(0);
            ra[t] = t < nval ? *reinterpret_cast<const Pk *>(gal + off) : one;
        }
        const uint16_t rb = gbe[hb + static_cast<int64_t>(min(t0 + (lane & 15), T - 1)) * H];
        const float bl = (lane & 15) < nval ? bf16_bits_to_f32(rb) : 0.f;  // beta of token lane & 15
        auto beta_of = [&](int t) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bl), t)); };
        // channel j of a packed pair, widened
        auto chan = [](Pk x, int j) { return bf16_bits_to_f32(static_cast<uint16_t>(x >> (16 * j))); };
        // CH consecutive bf16 of row t, channels CH*lane ..
        auto put = [&](__bf16 *m, int stride, int t, const float (&x)[CH]) {
            if constexpr (CH == 2) {
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                *reinterpret_cast<bf16x2 *>(m + t * stride + 2 * lane) = bf16x2{static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1])};
            } else {
                m[t * stride + lane] = static_cast<__bf16>(x[0]);
            }
        };
        // per-channel log2 decay prefix sums over the chunk
        float G[C16][CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < C16; ++t) {
                const float la = log2_decay(chan(ra[t], j));
                acc += la;
                G[t][j] = acc;
            }
        }
        // the other sub-chunk's log2 Gam_C: the odd one's from its decays (read
        // here, summed as its own pass sums them), the even one's kept
        float gpx[CH];
        if (!odd) {
            Pk rap[C16];
#pragma unroll
            for (int t = 0; t < C16; ++t)
                rap[t] = t < nval - C16 ? *reinterpret_cast<const Pk *>(gal + row(t0 + C16 + t)) : one;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int t = 0; t < C16; ++t) acc += log2_decay(chan(rap[t], j));
                gpx[j] = acc;
            }
        } else {
#pragma unroll
            for (int j = 0; j < CH; ++j) gpx[j] = gprev[j];
        }
        float gcx[CH], emax = 0.f;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            gcx[j] = G[C16 - 1][j];
            emax = fmaxf(emax, -gcx[j]);
        }
        // wave max of the largest exponent 2^{-G}
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) emax = fmaxf(emax, __shfl_xor(emax, m, 64));
        const bool fast = emax <= kFastLimit;
        float gcp[CH], gcq[CH];  // Gam_C per channel, own and the partner's
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            gcp[j] = exp2_fast(gcx[j]);
            gcq[j] = exp2_fast(gpx[j]);
        }
        // Tiles go to the block relative to the pair: the odd sub-chunk's k * Gam
        // and q * Gam also carry the even one's decay (they act on the state at
        // the pair start), the even sub-chunk's k * Gam_C / Gam also the odd
        // one's (it enters the state at the pair end).  Products within the
        // sub-chunk use the local tiles.
        float sdq[CH], se[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            sdq[j] = odd ? gcq[j] : 1.f;
            se[j] = odd ? 1.f : gcq[j];
        }
        // scaled tiles (the factored form's branch taken once per chunk): all
        // three go to the block, and the factored form also keeps k * Gam,
        // q * Gam and k / Gam in LDS for its products
        auto tiles = [&](auto fc) {
            constexpr bool F = decltype(fc)::value;
#pragma unroll
            for (int t = 0; t < C16; ++t) {
                float kd[CH], qd[CH], ke[CH], kb[CH];
#pragma unroll
                for (int j = 0; j < CH; ++j) {
                    const float kv = chan(rk[t], j), qv = chan(rq[t], j);
                    const float e1 = exp2_fast(G[t][j]);
                    kd[j] = kv * e1;
                    qd[j] = qv * e1;
                    if constexpr (F) {  // 2^{-G} is finite here: 2^{G_C - G} as a product
                        const float eb = exp2_fast(-G[t][j]);
                        kb[j] = kv * eb;
                        ke[j] = kv * (gcp[j] * eb);
                    } else {
                        kb[j] = 0.f;
                        ke[j] = kv * exp2_fast(gcx[j] - G[t][j]);
                    }
                }
                const float bt = beta_of(t);
                float kdo[CH], qdo[CH], keo[CH], keb[CH];
#pragma unroll
                for (int j = 0; j < CH; ++j) {
                    kdo[j] = kd[j] * sdq[j];
                    qdo[j] = qd[j] * sdq[j];
                    keb[j] = ke[j] * bt;
                    keo[j] = keb[j] * se[j];
                }
                put(o.kd, DK, t, kdo);
                put(o.qd, DK, t, qdo);
                put(o.ke, DK, t, keo);
                // local beta k * Gam_C / Gam for the odd sub-chunk's cross
                // blocks (their column scale diag(beta_0) comes with it)
                if (!odd) put(s.k0, KS, t, keb);
                if constexpr (F) {
                    put(s.a, KS, t, kd);
                    put(s.b, KS, t, qd);
                    put(s.kb, KS, t, kb);
                }
            }
        };
        if (fast) tiles(std::true_type{});
        else tiles(std::false_type{});
#pragma unroll
        for (int j = 0; j < CH; ++j) o.gc[CH * lane + j] = gcp[j] * gcq[j];  // the pair's (read from even blocks)
        if (lane < C16) s.beta[lane] = lane < nval ? bf16_bits_to_f32(rb) : 0.f;  // zero on padding rows
        wave_lds_fence();
        // Gram block G[t][s] (lane (g, i): t = 4g + r, s = i) and the
        // Aqk block as (K/Gam)(Q*Gam)^T (lane (g, i): s = 4g + r, t = i)
        f32x4 gr = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
        if (fast) {
#pragma unroll
            for (int p = 0; p < KSTEP; ++p) {
                const bf16x8 kdf = row_frag2(s.a, KS, 0, 32 * p, lane);
                const bf16x8 kbf = row_frag2(s.kb, KS, 0, 32 * p, lane);
                const bf16x8 qdf = row_frag2(s.b, KS, 0, 32 * p, lane);
                gr = mfma32(kdf, kbf, gr);
                aq = mfma32(kbf, qdf, aq);
            }
        } else {
            // Exact form for chunks whose decay leaves the factored range.
            // Entry (t, s), s < t, is formed at level b = highest set bit of
            // t ^ s: t and s then sit on either side of the reference token
            // m = (t & ~(2b - 1)) + b - 1, and
            //   2^{G_t - G_s} = 2^{G_t - G_m} 2^{G_m - G_s}
            // with both factors <= 1.  Each level is one masked product over
            // tiles whose rows are scaled against their own block's reference;
            // entries of other levels are discarded.  The last level (b = 0)
            // gives the diagonal of Aqk, undecayed.
            auto level = [&](auto bi) {
                constexpr int bl = decltype(bi)::value == 4 ? 0 : 8 >> decltype(bi)::value;
                auto row = [&](auto tc) {
                    constexpr int t = decltype(tc)::value;
                    float ak[CH], aqv[CH], bk[CH];
#pragma unroll
                    for (int j = 0; j < CH; ++j) {
                        const float kv = chan(rk[t], j), qv = chan(rq[t], j);
                        float rf = 1.f, cf = 1.f;
                        if constexpr (bl != 0) {
                            constexpr int m = (t & ~(2 * bl - 1)) + bl - 1;
                            if constexpr ((t & bl) != 0) {
                                rf = exp2_fast(G[t][j] - G[m][j]);
                                cf = 0.f;
                            } else {
                                rf = 0.f;
                                cf = exp2_fast(G[m][j] - G[t][j]);
                            }
                        }
                        ak[j] = kv * rf;
                        aqv[j] = qv * rf;
                        bk[j] = kv * cf;
                    }
                    if constexpr (bl != 0) put(s.a, KS, t, ak);
                    put(s.b, KS, t, aqv);
                    put(s.kb, KS, t, bk);
                };
                static_for<C16>(row);
                wave_lds_fence();
                f32x4 g2 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) {
                    const bf16x8 kbf = row_frag2(s.kb, KS, 0, 32 * p, lane);
                    if constexpr (bl != 0) g2 = mfma32(row_frag2(s.a, KS, 0, 32 * p, lane), kbf, g2);
                    a2 = mfma32(kbf, row_frag2(s.b, KS, 0, 32 * p, lane), a2);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int x = (4 * lg + r) ^ lc;  // same for both layouts
                    if constexpr (bl != 0) {
                        const bool at = x >= bl && x < 2 * bl;
                        if (at && ((4 * lg + r) & bl)) gr[r] = g2[r];  // t = 4g + r, s = i
                        if (at && (lc & bl)) aq[r] = a2[r];            // s = 4g + r, t = i
                    } else if (x == 0) {
                        aq[r] = a2[r];
                    }
                }
                wave_lds_fence();  // tiles are rewritten by the next level
                __builtin_amdgcn_sched_barrier(0);  // one level's values live at a time
            };
            static_for<5>(level);
        }
        // N diag(beta) = G beta_s (s < t) by column; Aqk diag(beta) (s <= t)
        {
            const float4 bt4 = *reinterpret_cast<const float4 *>(&s.beta[4 * lg]);
            const float bt[4] = {bt4.x, bt4.y, bt4.z, bt4.w};  // beta_s of Aqk's rows s = 4g + r
            const float bs = s.beta[lc];                         // beta_s of G's column s = i
            float l[4];
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                l[r] = lc < 4 * lg + r ? gr[r] * bs : 0.f;
                x[r] = 4 * lg + r <= lc ? aq[r] * bt[r] : 0.f;
            }
            *reinterpret_cast<float4 *>(&s.lt[lc * KLTS + 4 * lg]) = make_float4(l[0], l[1], l[2], l[3]);
            o.aqk[lane] = bf4(x);
        }
        wave_lds_fence();
        // D = (I + N diag(beta))^{-1}: forward substitution in fp32, lane = (column, row quad)
        {
            const int col = lane >> 2, q = lane & 3;
            float x[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (4 * q + r == col) ? 1.f : 0.f;
            auto sweep = [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const float4 l4 = *reinterpret_cast<const float4 *>(&s.lt[j * KLTS + 4 * q]);
                const float xj = quad_bcast<j / 4>(x[j % 4]);
                x[0] = fmaf(-l4.x, xj, x[0]);
                x[1] = fmaf(-l4.y, xj, x[1]);
                x[2] = fmaf(-l4.z, xj, x[2]);
                x[3] = fmaf(-l4.w, xj, x[3]);
            };
            static_for<15>(sweep);
            __bf16 *dt = reinterpret_cast<__bf16 *>(&s.dt[0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) dt[((col >> 2) * 16 + 4 * q + r) * 4 + (col & 3)] = static_cast<__bf16>(x[r]);
        }
        wave_lds_fence();
        o.dt[lane] = s.dt[lane];
#pragma unroll
        for (int j = 0; j < CH; ++j) gprev[j] = gcx[j];
        if (!odd) continue;
        // Cross blocks of the pair (odd sub-chunk t, even sub-chunk s): each
        // entry sum_c x_tc k_sc 2^{G_tc - G_sc} splits at the last even token
        // into 2^{G_tc} (this sub-chunk's own decay) and 2^{Gp_15c - Gp_sc} (the
        // even one's decay to its end), both at most 1, so the local tiles give
        // it exactly:  G_10 = (K_1 * Gam_1) (K_0 * Gam_C0 / Gam_0)^T and
        // Aqk_10 = (Q_1 * Gam_1) (K_0 * Gam_C0 / Gam_0)^T.
        wave_lds_fence();
#pragma unroll
        for (int t = 0; t < C16; ++t) {
            float kd[CH], qd[CH];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const float e1 = exp2_fast(G[t][j]);
                kd[j] = chan(rk[t], j) * e1;
                qd[j] = chan(rq[t], j) * e1;
            }
            put(s.a, KS, t, kd);
            put(s.b, KS, t, qd);
        }
        wave_lds_fence();
        f32x4 g10 = {0.f, 0.f, 0.f, 0.f}, a10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KSTEP; ++p) {
            const bf16x8 k0f = row_frag2(s.k0, KS, 0, 32 * p, lane);
            g10 = mfma32(row_frag2(s.a, KS, 0, 32 * p, lane), k0f, g10);  // lane (g, i): [t = 4g + r][s = i]
            a10 = mfma32(k0f, row_frag2(s.b, KS, 0, 32 * p, lane), a10);  // lane (g, i): [s = 4g + r][t = i]
        }
        o.ax[lane] = bf4(a10);
        // M_10 = -D_1 G_10 diag(beta_0) (the beta_0 came with the even
        // tile), formed transposed (A = -(G_10 diag(beta_0))^T from the
        // accumulator, B = D_1^T from its A-operand fragment) so it comes out
        // in A-operand order
        o.mx[lane] = bf4(mfma16(bf4(-g10), s.dt[lane], f32x4{0.f, 0.f, 0.f, 0.f}));
    }
}

// R of a pair of sub-chunks from the bf16 state at the pair start:
//   Z_i = (K*Gam)_i S^T (pair-relative tiles), R_0 = D_0 (V_0 - Z_0),
//   R_1 = D_1 (V_1 - Z_1) + M_10 R_0.
// The carry and the output wave both call this on the same operands, so both
// get the same R bit for bit.  Lane (g, i) holds rows t = 4g + r, column i.
template <int KSTEP, int KT>
__device__ __forceinline__ void pair_solve(const bf16x8 (&kf0)[KSTEP], const bf16x8 (&kf1)[KSTEP], const bf16x4 (&Sb)[KT],
                                           bf16x4 vb0, bf16x4 vb1, bf16x4 dt0, bf16x4 dt1, bf16x4 mxf, bf16x4 &ub0,
                                           bf16x4 &ub1) {
    f32x4 z00 = {0.f, 0.f, 0.f, 0.f}, z01 = {0.f, 0.f, 0.f, 0.f};
    f32x4 z10 = {0.f, 0.f, 0.f, 0.f}, z11 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KSTEP; p += 2) {  // two independent accumulation chains per sub-chunk
        const bf16x8 b0 = cat8(Sb[2 * p], Sb[2 * p + 1]), b1 = cat8(Sb[2 * p + 2], Sb[2 * p + 3]);
        z00 = mfma32(kf0[p], b0, z00);
        z01 = mfma32(kf0[p + 1], b1, z01);
        z10 = mfma32(kf1[p], b0, z10);
        z11 = mfma32(kf1[p + 1], b1, z11);
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 r0 = __builtin_convertvector(vb0, f32x4) - (z00 + z01);
    const f32x4 r1 = __builtin_convertvector(vb1, f32x4) - (z10 + z11);
    const f32x4 u0 = mfma16(dt0, bf4(r0), zero);
    const f32x4 u1 = mfma16(dt1, bf4(r1), zero);
    ub0 = bf4(u0);
    ub1 = bf4(mfma16(mxf, ub0, u1));
}

template <int DK, int NVT, bool SIDE>
__global__ __launch_bounds__(KdaShape<NVT>::NT) void kda_chunked_kernel(DeltaArgs a, const KdaBlock<DK> *__restrict__ der,
                                                                         int64_t Ts, int64_t tb, unsigned int *status) {
    constexpr int KBV = KdaShape<NVT>::BV;
    constexpr int KS = DK + 8, VS = KBV + 8;
    constexpr int KSTEP = DK / 32, KT = DK / 16;
    using Lds = KdaLds<DK, NVT>;
    __shared__ Lds s;

    const int T = static_cast<int>(a.T), H = static_cast<int>(a.H), dv = a.dv;
    int head, slice;
    xcd_group_map(blockIdx.x, static_cast<int>(a.B * a.H), dv / KBV, head, slice);
    const int b = head / H, h = head % H;
    const int v0 = slice * KBV;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lg = lane >> 4, lc = lane & 15;
    const int npairs = (T + 2 * C16 - 1) / (2 * C16);  // steps of two 16-token sub-chunks
    auto tok = [&](int t) { return (static_cast<int64_t>(b) * Ts + tb + t) * H + h; };

    if (tid == 0) {
        for (int i = 0; i < NSLOT; ++i) s.ready[i] = 0u;
        for (int i = 0; i < NVT; ++i) s.cons[i] = s.sp[i] = s.so[i] = 0u;
    }
    __syncthreads();

    if (wave < 2 * NVT) {
        const int vt = wave % NVT;
        const int vcol = v0 + 16 * vt + lc;
        const int64_t sbase = (static_cast<int64_t>(head) * dv + vcol) * DK;
        if (wave < NVT) {
            // ================================ carry ================================
            f32x4 St[KT];
            if (a.state_in) {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    const float4 x = *reinterpret_cast<const float4 *>(a.state_in + sbase + 16 * kt + 4 * lg);
                    St[kt] = f32x4{x.x, x.y, x.z, x.w};
                }
            } else {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) St[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) s.sh[0][vt][kt][lane] = bf4(St[kt]);
            lds_arrive(&s.sp[vt], lane);
            // Operands of a pair that do not depend on the state, read one
            // pair ahead: the next slot's reads go out while this pair's
            // state-update products run.
            bf16x8 kf0[KSTEP], kf1[KSTEP], kef[KT];
            bf16x4 vb0, vb1, dt0, dt1, mxf;
            float4 gcv[KT];
            auto load_ops = [&](int c) {
                const typename Lds::Slot &Sl = s.slot[c & 3];
                lds_wait(&s.ready[c & 3], static_cast<unsigned int>(c / 4 + 1), status);
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) {
                    kf0[p] = row_frag2(Sl.kd, KS, 0, 32 * p, lane);
                    kf1[p] = row_frag2(Sl.kd, KS, C16, 32 * p, lane);
                }
                vb0 = col_gather4(Sl.v, VS, 0, 16 * vt, lane);
                vb1 = col_gather4(Sl.v, VS, C16, 16 * vt, lane);
                dt0 = Sl.dt[0][lane];
                dt1 = Sl.dt[1][lane];
                mxf = Sl.mx[lane];
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    kef[kt] = col_frag(Sl.ke, KS, 0, 16 * kt, lane);
                    gcv[kt] = *reinterpret_cast<const float4 *>(&Sl.gc[16 * kt + 4 * lg]);
                }
            };
            // bf16 copy of the state: B operand of the next Z and the output's copy
            bf16x4 Sb[KT];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) Sb[kt] = bf4(St[kt]);
            if (npairs > 0) load_ops(0);
#pragma unroll 1
            for (int c = 0; c < npairs; ++c) {
                bf16x4 ub0, ub1;
                pair_solve(kf0, kf1, Sb, vb0, vb1, dt0, dt1, mxf, ub0, ub1);
                // S^T <- diag(Gam_C) S^T + [beta K*Gam_C/Gam]^T [R_0; R_1] over the 32 tokens
                const bf16x8 bU = cat8(ub0, ub1);
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    St[kt] = St[kt] * f32x4{gcv[kt].x, gcv[kt].y, gcv[kt].z, gcv[kt].w};
                    St[kt] = mfma32(kef[kt], bU, St[kt]);
                }
                if constexpr (SIDE) {  // routing signal: the residuals (bf16, as carried) or the targets
                    const bool res = a.side_kind == kSideResidual;
                    uint16_t *so = static_cast<uint16_t *>(a.side) + vcol;
                    const uint2 x0 = __builtin_bit_cast(uint2, ub0), y0 = __builtin_bit_cast(uint2, vb0);
                    const uint2 x1 = __builtin_bit_cast(uint2, ub1), y1 = __builtin_bit_cast(uint2, vb1);
                    const uint32_t w[4] = {res ? x0.x : y0.x, res ? x0.y : y0.y, res ? x1.x : y1.x, res ? x1.y : y1.y};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {  // sub-chunk e / 4, row 4 lg + e % 4
                        const int t = 2 * C16 * c + C16 * (e >> 2) + 4 * lg + (e & 3);
                        const uint32_t w2 = w[e >> 1];
                        if (t < T) so[tok(t) * dv] = static_cast<uint16_t>(e & 1 ? w2 >> 16 : w2);
                    }
                }
                if (c + 1 < npairs) load_ops(c + 1);
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) Sb[kt] = bf4(St[kt]);
                // S(c + 1 - NSB) has been read from this buffer
                if constexpr (Lds::kStateGuard) lds_wait(&s.so[vt], static_cast<unsigned int>(c + 2 - Lds::NSB), status);
                {
                    auto &dst = s.sh[(c + 1) % Lds::NSB][vt];
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) dst[kt][lane] = Sb[kt];
                }
                lds_arrive(&s.sp[vt], lane);  // also releases slot c: its last read precedes this
            }
            if (a.state_out) {
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
                    *reinterpret_cast<float4 *>(a.state_out + sbase + 16 * kt + 4 * lg) =
                        make_float4(St[kt][0], St[kt][1], St[kt][2], St[kt][3]);
            }
        } else {
            // ================================ output ===============================
            for (int c = 0; c < npairs; ++c) {
                const typename Lds::Slot &Sl = s.slot[c & 3];
                lds_wait(&s.ready[c & 3], static_cast<unsigned int>(c / 4 + 1), status);
                // state-independent operands first
                bf16x8 qf0[KSTEP], qf1[KSTEP], kf0[KSTEP], kf1[KSTEP];
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) {
                    qf0[p] = row_frag2(Sl.qd, KS, 0, 32 * p, lane);
                    qf1[p] = row_frag2(Sl.qd, KS, C16, 32 * p, lane);
                    kf0[p] = row_frag2(Sl.kd, KS, 0, 32 * p, lane);
                    kf1[p] = row_frag2(Sl.kd, KS, C16, 32 * p, lane);
                }
                const bf16x4 aq0 = Sl.aqk[0][lane], aq1 = Sl.aqk[1][lane], axf = Sl.ax[lane];
                const bf16x4 vb0 = col_gather4(Sl.v, VS, 0, 16 * vt, lane);
                const bf16x4 vb1 = col_gather4(Sl.v, VS, C16, 16 * vt, lane);
                const bf16x4 dt0 = Sl.dt[0][lane], dt1 = Sl.dt[1][lane], mxf = Sl.mx[lane];
                lds_wait(&s.sp[vt], static_cast<unsigned int>(c + 1), status);
                bf16x4 Sb[KT];
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) Sb[kt] = s.sh[c % Lds::NSB][vt][kt][lane];
                if constexpr (Lds::kStateGuard) lds_arrive(&s.so[vt], lane);
                // R exactly as the carry forms it, from the same bf16 state
                bf16x4 ub0, ub1;
                pair_solve(kf0, kf1, Sb, vb0, vb1, dt0, dt1, mxf, ub0, ub1);
                // Y^T = S (Q*Gam)^T + R^T Aqk^T: lane (g, i) holds columns 4g + r of
                // token i; two independent accumulation chains per sub-chunk
                f32x4 y00 = {0.f, 0.f, 0.f, 0.f}, y01 = {0.f, 0.f, 0.f, 0.f};
                f32x4 y10 = {0.f, 0.f, 0.f, 0.f}, y11 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KSTEP; p += 2) {
                    const bf16x8 b0 = cat8(Sb[2 * p], Sb[2 * p + 1]), b1 = cat8(Sb[2 * p + 2], Sb[2 * p + 3]);
                    y00 = mfma32(b0, qf0[p], y00);
                    y01 = mfma32(b1, qf0[p + 1], y01);
                    y10 = mfma32(b0, qf1[p], y10);
                    y11 = mfma32(b1, qf1[p + 1], y11);
                }
                const f32x4 y0 = mfma16(ub0, aq0, y00 + y01);
                const f32x4 y1 = mfma16(ub1, aq1, mfma16(ub0, axf, y10 + y11));
                const int t = c * (2 * C16) + lc;
                uint16_t *yo = static_cast<uint16_t *>(a.out) + v0 + 16 * vt + 4 * lg;
                if (t < T) *reinterpret_cast<bf16x4 *>(yo + tok(t) * dv) = bf4(y0);
                if (t + C16 < T) *reinterpret_cast<bf16x4 *>(yo + tok(t + C16) * dv) = bf4(y1);
                lds_arrive(&s.cons[vt], lane);
            }
        }
    } else {
        // ============================== producers ==============================
        // Producer pw copies pairs pw, pw + 4, ...: the pair's two blocks,
        // 16-byte piece p = 64i + lane per load, and the slice's 32 value rows
        // (KBV/8 lanes per row, 8 columns each).
        const int pw = wave - 2 * NVT;
        typename Lds::Slot &Sl = s.slot[pw];
        using Blk = KdaBlock<DK>;
        constexpr int NP2 = 2 * Blk::kPieces;          // pieces of the two blocks of a pair
        constexpr int NPL = (NP2 + 63) / 64;           // pieces per lane
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 *gder = reinterpret_cast<const u32x4 *>(der + static_cast<int64_t>(head) * 2 * npairs);
        const uint16_t *gv = static_cast<const uint16_t *>(a.v);
        constexpr int VLPR = KBV / 8;                  // lanes per value row
        constexpr int VRPL = 64 / VLPR;                // value rows per load
        constexpr int NVL = 2 * C16 / VRPL;            // value loads per pair
        const int vrow = lane / VLPR, vcol = 8 * (lane % VLPR);
        u32x4 rd[NPL];
        uint4 rv[NVL];
        int nnext = 0;  // tokens inside the sequence from the staged pair's start
        auto fetch = [&](int n) {
            const u32x4 *src = gder + static_cast<int64_t>(n) * (2 * sizeof(Blk) / 16);
#pragma unroll
            for (int i = 0; i < NPL; ++i) rd[i] = src[min(64 * i + lane, NP2 - 1)];
            const int t0 = n * 2 * C16;
            nnext = T - t0;
#pragma unroll
            for (int j = 0; j < NVL; ++j)
                rv[j] = *reinterpret_cast<const uint4 *>(gv + tok(min(t0 + vrow + VRPL * j, T - 1)) * dv + v0 + vcol);
        };
        // LDS place of piece p: token-row pieces go to padded rows (the odd
        // block's below the even one's); the even block supplies the pair's
        // Gam_C, the odd block the cross blocks
        auto commit = [&](int nval) {
            constexpr int PPR = DK / 8;  // pieces per row
#pragma unroll
            for (int i = 0; i < NPL; ++i) {
                const int p = 64 * i + lane;
                if (p >= NP2) continue;
                const int blk = p >= Blk::kPieces ? 1 : 0;
                const int q = p - blk * Blk::kPieces;
                if (q < Blk::kRowPieces) {
                    const int r = q / PPR;       // row among the 3 * 16 of the block
                    const int tsr = r / C16;     // kd, ke, qd
                    __bf16 *rows = tsr == 0 ? Sl.kd : (tsr == 1 ? Sl.ke : Sl.qd);
                    *reinterpret_cast<u32x4 *>(rows + (C16 * blk + r % C16) * KS + 8 * (q % PPR)) = rd[i];
                } else {
                    const int e = q - Blk::kRowPieces;
                    if (e < 32) {
                        reinterpret_cast<u32x4 *>(&Sl.aqk[blk][0])[e] = rd[i];
                    } else if (e < 64) {
                        reinterpret_cast<u32x4 *>(&Sl.dt[blk][0])[e - 32] = rd[i];
                    } else if (e < 64 + DK / 4) {
                        if (blk == 0) reinterpret_cast<u32x4 *>(&Sl.gc[0])[e - 64] = rd[i];
                    } else if (blk == 1) {
                        const int x = e - 64 - DK / 4;
                        if (x < 32) reinterpret_cast<u32x4 *>(&Sl.mx[0])[x] = rd[i];
                        else reinterpret_cast<u32x4 *>(&Sl.ax[0])[x - 32] = rd[i];
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < NVL; ++j) {
                const int row = vrow + VRPL * j;
                const uint32_t m = row < nval ? 0xffffffffu : 0u;
                *reinterpret_cast<uint4 *>(&Sl.v[row * VS + vcol]) =
                    make_uint4(rv[j].x & m, rv[j].y & m, rv[j].z & m, rv[j].w & m);
            }
        };
        if (pw < npairs) fetch(pw);
        for (int n = pw; n < npairs; n += 4) {
            const int nval = nnext;
            if (n >= 4) {  // pair n - 4 released by every consumer wave
#pragma unroll
                for (int w = 0; w < NVT; ++w) {
                    lds_wait(&s.sp[w], static_cast<unsigned int>(n - 2), status);    // carry w past pair n - 4
                    lds_wait(&s.cons[w], static_cast<unsigned int>(n - 3), status);  // output w done with it
                }
            }
            commit(nval);
            lds_arrive(&s.ready[pw], lane);
            // this producer's next pair (past the end: the last pair again, unused)
            fetch(min(n + 4, npairs - 1));
        }
    }
}

}  // namespace

bool kda_chunked_supported(const DeltaArgs &a) {
    return a.variant == kKimiDelta && a.dtype == kBF16 && (a.dk == 64 || a.dk == 128) && a.dv % 16 == 0;
}

bool kda_chunked_workspace(const DeltaArgs &a, size_t *bytes) {
    const int64_t tasks = 2 * a.B * a.H * ((a.T + 2 * C16 - 1) / (2 * C16));  // blocks (sub-chunks)
    if (tasks > 0x7fffffff) return false;
    const size_t blk = a.dk == 64 ? sizeof(KdaBlock<64>) : sizeof(KdaBlock<128>);
    *bytes = kStatusBytes + static_cast<size_t>(tasks) * blk;
    return true;
}

template <int DK, int NVT>
static hipError_t launch_dk(const DeltaArgs &a, hipStream_t stream) {
    const unsigned blocks = static_cast<unsigned>(a.B * a.H * (a.dv / KdaShape<NVT>::BV));
    const int64_t np = (a.T + 2 * C16 - 1) / (2 * C16);  // pairs per sequence
    const int64_t pairs = a.B * a.H * np;                // derivation waves
    unsigned int *status = static_cast<unsigned int *>(a.ws);
    KdaBlock<DK> *der = reinterpret_cast<KdaBlock<DK> *>(static_cast<char *>(a.ws) + kStatusBytes);
    if (pairs > 0)
        kda_derive_kernel<DK><<<static_cast<unsigned>(pairs), 64, 0, stream>>>(a, der, a.T, 0, status);
    if (a.side)
        kda_chunked_kernel<DK, NVT, true><<<blocks, KdaShape<NVT>::NT, 0, stream>>>(a, pairs > 0 ? der : nullptr, a.T, 0, status);
    else
        kda_chunked_kernel<DK, NVT, false><<<blocks, KdaShape<NVT>::NT, 0, stream>>>(a, pairs > 0 ? der : nullptr, a.T, 0, status);
    return hipGetLastError();
}

template <int NVT>
static hipError_t launch_nvt(const DeltaArgs &a, hipStream_t stream) {
    switch (a.dk) {
        case 64: return launch_dk<64, NVT>(a, stream);
        case 128: return launch_dk<128, NVT>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

// Two value tiles per workgroup share the producers' work; with fewer than
// 256 such workgroups the chip has idle compute units, and one tile per
// workgroup doubles the number of chains running at once.
hipError_t launch_kda_chunked(const DeltaArgs &a, hipStream_t stream) {
    if (!kda_chunked_supported(a)) return hipErrorNotSupported;
    if (a.dv % 32 == 0 && a.B * a.H * (a.dv / 32) >= 256) return launch_nvt<2>(a, stream);
    return launch_nvt<1>(a, stream);
}

}  // namespace lam
