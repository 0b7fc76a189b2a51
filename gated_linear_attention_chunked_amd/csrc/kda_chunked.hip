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
//   L   = strict_lower(diag(beta) ((K * Gam) (K / Gam)^T))
//   U   = (I + L)^{-1} diag(beta) (V - (K * Gam) S^T)
//   Y   = (Q * Gam) S^T + lower((Q * Gam) (K / Gam)^T) U
//   S'  = S diag(Gam_C) + U^T (K * Gam_C / Gam)
// Every entry of the two Gram-type products is sum_c x_tc k_sc 2^{G_tc - G_sc}
// with s <= t, at most |x_t||k_s|.  Splitting 2^{G_t - G_s} into 2^{G_t} and
// 2^{-G_s} puts both products on MFMA; 2^{-G_s} stays finite while the decay
// over the chunk keeps every channel above 2^-100.  A chunk that decays
// further (alpha near zero somewhere) takes an exact path instead: each entry
// is summed channel by channel with 2^{G_tc - G_sc} <= 1 evaluated directly.
// C = 16 makes the Gram a single 16x16 block, so one factorisation serves the
// whole chunk.
//
// Schedule: one workgroup of 8 waves per (b, h, 32-column value slice).
//   carry  (waves 0-1, one 16-column tile each): Z = (K*Gam) S^T, the 16x16
//          solve on one MFMA, U published, state update S^T <- diag(Gam_C)
//          S^T + (K*Gam_C/Gam)^T U, bf16 copy of S published for the output.
//   output (waves 2-3): Y^T = S (Q*Gam)^T + U^T Aqk^T, 8-byte row stores.
//   producers (waves 4-7): producer p derives every fourth chunk (p, p+4, ...)
//          into its own LDS slot: loads one chunk ahead in registers, the
//          per-channel prefix sums and powers of two (lane = channel pair),
//          the scaled key/query tiles, the Gram and Aqk blocks, the fp32
//          inverse of I + L and D diag(beta).
// There is no workgroup barrier in the chunk loop: slots, U and the bf16
// state move between roles through bounded LDS counters.
#include <type_traits>

#include "chunk_common.h"
#include "lam_internal.h"

namespace lam {
namespace {

constexpr int C16 = 16;      // chunk length (tokens)
constexpr int NSLOT = 4;     // one derived-chunk slot per producer
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

template <int DK, int NVT>
struct KdaLds {
    static constexpr int KS = DK + 8;
    static constexpr int VS = KdaShape<NVT>::BV + 8;
    struct Slot {  // state-independent data of one chunk
        alignas(16) __bf16 kd[C16 * KS];   // k * Gam
        alignas(16) __bf16 ke[C16 * KS];   // k * Gam_C / Gam
        alignas(16) __bf16 qd[C16 * KS];   // q * Gam
        alignas(16) __bf16 v[C16 * VS];    // value targets of the workgroup's columns
        alignas(16) bf16x4 aqk[64];        // lower((Q*Gam)(K/Gam)^T), B-operand order: lane (g, i) holds [t = i][s = 4g + r]
        alignas(16) bf16x4 dt[64];         // (I + L)^{-1} diag(beta), A-operand order
        alignas(16) float gc[DK];          // Gam_C per channel
    };
    struct Scratch {  // per producer
        alignas(16) __bf16 kb[C16 * KS];   // k / Gam (factored form); column tile (exact form)
        alignas(16) __bf16 ka[C16 * KS];   // exact form: row tiles of k and q
        alignas(16) __bf16 qa[C16 * KS];
        alignas(16) float lt[16 * KLTS];   // L by column
        alignas(16) float beta[C16];
    };
    Slot slot[NSLOT];
    Scratch scr[4];
    // A producer publishes chunk c only after every consumer has finished
    // chunk c - 4, so the carry can run at most four chunks ahead of the
    // output: four U buffers need no further check, and with five state
    // buffers neither does the bf16 state (two when LDS is short, guarded by
    // the output's read count).
    static constexpr int NUB = 4;
    static constexpr int NSB = NVT == 1 ? 5 : 2;
    static constexpr bool kStateGuard = NSB < 5;
    alignas(16) bf16x4 uh[NUB][NVT][64];           // U per chunk and tile
    alignas(16) bf16x4 sh[NSB][NVT][DK / 16][64];  // bf16 state per chunk and tile
    unsigned int ready[NSLOT];   // chunks published per slot
    unsigned int cons[NVT];      // chunks finished per output wave
    unsigned int uc[NVT];        // U published per tile
    unsigned int sp[NVT], so[NVT];   // bf16 state published / read per tile
};

template <int DK, int NVT>
__global__ __launch_bounds__(KdaShape<NVT>::NT) void kda_chunked_kernel(DeltaArgs a) {
    constexpr int KBV = KdaShape<NVT>::BV;
    constexpr int KS = DK + 8, VS = KBV + 8;
    constexpr int KSTEP = DK / 32, KT = DK / 16, CH = DK / 64;  // CH: key channels per producer lane
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
    const int nchunks = (T + C16 - 1) / C16;
    auto tok = [&](int t) { return (static_cast<int64_t>(b) * T + t) * H + h; };

    if (tid == 0) {
        for (int i = 0; i < NSLOT; ++i) s.ready[i] = 0u;
        for (int i = 0; i < NVT; ++i) s.cons[i] = s.uc[i] = s.sp[i] = s.so[i] = 0u;
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
#pragma unroll 1
            for (int c = 0; c < nchunks; ++c) {
                const typename Lds::Slot &Sl = s.slot[c & 3];
                lds_wait(&s.ready[c & 3], static_cast<unsigned int>(c / 4 + 1));
                bf16x8 kf[KSTEP];
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) kf[p] = row_frag2(Sl.kd, KS, 0, 32 * p, lane);
                const bf16x4 vb = col_gather4(Sl.v, VS, 0, 16 * vt, lane);
                const bf16x4 dtf = Sl.dt[lane];
                // Z = (K*Gam) S^T: lane (g, i) holds rows t = 4g + r, column i
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) z = mfma32(kf[p], cat8(bf4(St[2 * p]), bf4(St[2 * p + 1])), z);
                const f32x4 rhs = __builtin_convertvector(vb, f32x4) - z;
                const bf16x4 ub = bf4(mfma16(dtf, bf4(rhs), f32x4{0.f, 0.f, 0.f, 0.f}));
                s.uh[c & 3][vt][lane] = ub;
                lds_arrive(&s.uc[vt], lane);
                // S^T <- diag(Gam_C) S^T + (K*Gam_C/Gam)^T U
                bf16x4 kef[KT];
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) kef[kt] = col_gather4(Sl.ke, KS, 0, 16 * kt, lane);
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    const float4 g4 = *reinterpret_cast<const float4 *>(&Sl.gc[16 * kt + 4 * lg]);
                    St[kt] = St[kt] * f32x4{g4.x, g4.y, g4.z, g4.w};
                    St[kt] = mfma16(kef[kt], ub, St[kt]);
                }
                // S(c + 1 - NSB) has been read from this buffer
                if constexpr (Lds::kStateGuard) lds_wait(&s.so[vt], static_cast<unsigned int>(c + 2 - Lds::NSB));
                {
                    auto &dst = s.sh[(c + 1) % Lds::NSB][vt];
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) dst[kt][lane] = bf4(St[kt]);
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
            for (int c = 0; c < nchunks; ++c) {
                const typename Lds::Slot &Sl = s.slot[c & 3];
                lds_wait(&s.ready[c & 3], static_cast<unsigned int>(c / 4 + 1));
                lds_wait(&s.sp[vt], static_cast<unsigned int>(c + 1));
                bf16x8 bS[KSTEP];
#pragma unroll
                for (int p = 0; p < KSTEP; ++p)
                    bS[p] = cat8(s.sh[c % Lds::NSB][vt][2 * p][lane], s.sh[c % Lds::NSB][vt][2 * p + 1][lane]);
                if constexpr (Lds::kStateGuard) lds_arrive(&s.so[vt], lane);
                // Y^T = S (Q*Gam)^T + U^T Aqk^T: lane (g, i) holds columns 4g + r of token i
                f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) y = mfma32(bS[p], row_frag2(Sl.qd, KS, 0, 32 * p, lane), y);
                const bf16x4 aq = Sl.aqk[lane];
                lds_wait(&s.uc[vt], static_cast<unsigned int>(c + 1));
                const bf16x4 ub = s.uh[c & 3][vt][lane];
                y = mfma16(ub, aq, y);
                const int t = c * C16 + lc;
                if (t < T)
                    *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(a.out) + tok(t) * dv + v0 + 16 * vt + 4 * lg) = bf4(y);
                lds_arrive(&s.cons[vt], lane);
            }
        }
    } else {
        // ============================== producers ==============================
        const int pw = wave - 2 * NVT;
        typename Lds::Scratch &X = s.scr[pw];
        typename Lds::Slot &Sl = s.slot[pw];
        const uint16_t *gq = static_cast<const uint16_t *>(a.q);
        const uint16_t *gk = static_cast<const uint16_t *>(a.k);
        const uint16_t *gv = static_cast<const uint16_t *>(a.v);
        const uint16_t *gal = static_cast<const uint16_t *>(a.alpha);
        const uint16_t *gbe = static_cast<const uint16_t *>(a.beta);
        // Staged chunk: lane owns key channels CH*lane .. CH*lane + CH - 1
        // (one packed load per token and tensor) for all 16 tokens; value
        // row lane/4, columns 8 (lane % 4) ..; beta of token lane (lanes 0-15).
        using Pk = std::conditional_t<CH == 2, uint32_t, uint16_t>;
        Pk rk[C16], rq[C16], ra[C16];
        // value rows: KBV/8 lanes per row, 8 columns each (lanes past row 15 idle)
        constexpr int VLPR = KBV / 8;
        const int vrow = lane / VLPR, vcol = 8 * (lane % VLPR);
        uint4 rv;
        uint16_t rb = 0;
        int nval = 0, nnext = 0;  // tokens inside the sequence: chunk being derived, staged chunk
        // fetch_kq: keys and queries (the bulk); fetch_rest: decays, value
        // rows and beta.  Both clamp rows to the sequence.  A row's offset is
        // the same for the whole wave (scalar arithmetic); only the lane's
        // channel offset is per lane.
        const int64_t hdk = static_cast<int64_t>(H) * DK;
        const uint16_t *lk = gk + CH * lane, *lq = gq + CH * lane, *la = gal + CH * lane;
        auto fetch_kq = [&](int n) {
            const int t0 = n * C16, nn = min(C16, T - t0);
            const int64_t r0 = tok(t0) * DK;
#pragma unroll
            for (int t = 0; t < C16; ++t) {
                const int64_t o = r0 + min(t, nn - 1) * hdk;
                rk[t] = *reinterpret_cast<const Pk *>(lk + o);
                rq[t] = *reinterpret_cast<const Pk *>(lq + o);
            }
        };
        auto fetch_rest = [&](int n) {
            const int t0 = n * C16;
            nnext = min(C16, T - t0);
            const int64_t r0 = tok(t0) * DK;
#pragma unroll
            for (int t = 0; t < C16; ++t) ra[t] = *reinterpret_cast<const Pk *>(la + r0 + min(t, nnext - 1) * hdk);
            rv = *reinterpret_cast<const uint4 *>(gv + tok(t0 + min(vrow, nnext - 1)) * dv + v0 + vcol);
            if (lane < C16) rb = gbe[tok(t0 + min(lane, nnext - 1))];
        };
        // channel j of a packed pair, widened
        auto chan = [](Pk x, int j) { return bf16_bits_to_f32(static_cast<uint16_t>(x >> (16 * j))); };
        // CH consecutive bf16 of row t, channels CH*lane ..
        auto put = [&](__bf16 *m, int t, const float (&x)[CH]) {
            if constexpr (CH == 2) {
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                *reinterpret_cast<bf16x2 *>(m + t * KS + 2 * lane) = bf16x2{static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1])};
            } else {
                m[t * KS + lane] = static_cast<__bf16>(x[0]);
            }
        };
        if (pw < nchunks) {
            fetch_kq(pw);
            fetch_rest(pw);
        }
        for (int n = pw; n < nchunks; n += 4) {
            nval = nnext;
            if (n >= 4) {  // chunk n - 4 released by every consumer wave
#pragma unroll
                for (int w = 0; w < NVT; ++w) {
                    lds_wait(&s.sp[w], static_cast<unsigned int>(n - 2));    // carry w past chunk n - 4
                    lds_wait(&s.cons[w], static_cast<unsigned int>(n - 3));  // output w done with it
                }
            }
            // padding rows: zero key and query, decay 1
            if (nval < C16) {
                const Pk one = CH == 2 ? Pk(0x3f803f80u) : Pk(0x3f80u);
#pragma unroll
                for (int t = 0; t < C16; ++t) {
                    if (t >= nval) {
                        rk[t] = 0;
                        rq[t] = 0;
                        ra[t] = one;
                    }
                }
            }
            // per-channel log2 decay prefix sums over the chunk
            float G[C16][CH];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int t = 0; t < C16; ++t) {
                    const float la = fmaxf(__builtin_amdgcn_logf(chan(ra[t], j)), -200.f);
                    acc += la;
                    G[t][j] = acc;
                }
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
            float gcp[CH];  // Gam_C per channel
#pragma unroll
            for (int j = 0; j < CH; ++j) gcp[j] = exp2_fast(gcx[j]);
            // scaled tiles (the factored form's branch taken once per chunk)
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
                    put(Sl.kd, t, kd);
                    put(Sl.qd, t, qd);
                    put(Sl.ke, t, ke);
                    if constexpr (F) put(X.kb, t, kb);
                }
            };
            if (fast) tiles(std::true_type{});
            else tiles(std::false_type{});
#pragma unroll
            for (int j = 0; j < CH; ++j) Sl.gc[CH * lane + j] = gcp[j];
            {
                const uint32_t m = vrow < nval ? 0xffffffffu : 0u;
                if (vrow < C16)
                    *reinterpret_cast<uint4 *>(&Sl.v[vrow * VS + vcol]) = make_uint4(rv.x & m, rv.y & m, rv.z & m, rv.w & m);
            }
            if (lane < C16) X.beta[lane] = lane < nval ? bf16_bits_to_f32(rb) : 0.f;
            wave_lds_fence();
            // Gram block G[t][s] (lane (g, i): t = 4g + r, s = i) and the
            // Aqk block as (K/Gam)(Q*Gam)^T (lane (g, i): s = 4g + r, t = i)
            f32x4 gr = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
            if (fast) {
#pragma unroll
                for (int p = 0; p < KSTEP; ++p) {
                    const bf16x8 kdf = row_frag2(Sl.kd, KS, 0, 32 * p, lane);
                    const bf16x8 kbf = row_frag2(X.kb, KS, 0, 32 * p, lane);
                    const bf16x8 qdf = row_frag2(Sl.qd, KS, 0, 32 * p, lane);
                    gr = mfma32(kdf, kbf, gr);
                    aq = mfma32(kbf, qdf, aq);
                }
            } else {
                // Exact form for chunks whose decay leaves the factored range.
                // Entry (t, s), s < t, is formed at level b = highest set bit
                // of t ^ s: t and s then sit on either side of the reference
                // token m = (t & ~(2b - 1)) + b - 1, and
                //   2^{G_t - G_s} = 2^{G_t - G_m} 2^{G_m - G_s}
                // with both factors <= 1.  Each level is one masked product
                // over tiles whose rows are scaled against their own block's
                // reference; entries of other levels are discarded.  The last
                // level (b = 0) gives the diagonal of Aqk, undecayed.
                auto level = [&](auto bi) {
                    constexpr int b = decltype(bi)::value == 4 ? 0 : 8 >> decltype(bi)::value;
                    auto row = [&](auto tc) {
                        constexpr int t = decltype(tc)::value;
                        float ak[CH], aqv[CH], bk[CH];
#pragma unroll
                        for (int j = 0; j < CH; ++j) {
                            const float kv = chan(rk[t], j), qv = chan(rq[t], j);
                            float rf = 1.f, cf = 1.f;
                            if constexpr (b != 0) {
                                constexpr int m = (t & ~(2 * b - 1)) + b - 1;
                                if constexpr ((t & b) != 0) {
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
                        if constexpr (b != 0) put(X.ka, t, ak);
                        put(X.qa, t, aqv);
                        put(X.kb, t, bk);
                    };
                    static_for<C16>(row);
                    wave_lds_fence();
                    f32x4 g2 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int p = 0; p < KSTEP; ++p) {
                        const bf16x8 kbf = row_frag2(X.kb, KS, 0, 32 * p, lane);
                        if constexpr (b != 0) g2 = mfma32(row_frag2(X.ka, KS, 0, 32 * p, lane), kbf, g2);
                        a2 = mfma32(kbf, row_frag2(X.qa, KS, 0, 32 * p, lane), a2);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int x = (4 * lg + r) ^ lc;  // same for both layouts
                        if constexpr (b != 0) {
                            const bool at = x >= b && x < 2 * b;
                            if (at && ((4 * lg + r) & b)) gr[r] = g2[r];  // t = 4g + r, s = i
                            if (at && (lc & b)) aq[r] = a2[r];            // s = 4g + r, t = i
                        } else if (x == 0) {
                            aq[r] = a2[r];
                        }
                    }
                    wave_lds_fence();  // tiles are rewritten by the next level
                    __builtin_amdgcn_sched_barrier(0);  // one level's values live at a time
                };
                static_for<5>(level);
            }
            // L = beta_t G (s < t) by column; Aqk (s <= t)
            {
                const float4 bt4 = *reinterpret_cast<const float4 *>(&X.beta[4 * lg]);
                const float bt[4] = {bt4.x, bt4.y, bt4.z, bt4.w};
                float l[4];
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    l[r] = lc < 4 * lg + r ? bt[r] * gr[r] : 0.f;
                    x[r] = 4 * lg + r <= lc ? aq[r] : 0.f;
                }
                *reinterpret_cast<float4 *>(&X.lt[lc * KLTS + 4 * lg]) = make_float4(l[0], l[1], l[2], l[3]);
                Sl.aqk[lane] = bf4(x);
            }
            wave_lds_fence();
            // D = (I + L)^{-1}: forward substitution in fp32, lane = (column, row quad)
            {
                const int col = lane >> 2, q = lane & 3;
                float x[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = (4 * q + r == col) ? 1.f : 0.f;
                auto sweep = [&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    const float4 l4 = *reinterpret_cast<const float4 *>(&X.lt[j * KLTS + 4 * q]);
                    const float xj = quad_bcast<j / 4>(x[j % 4]);
                    x[0] = fmaf(-l4.x, xj, x[0]);
                    x[1] = fmaf(-l4.y, xj, x[1]);
                    x[2] = fmaf(-l4.z, xj, x[2]);
                    x[3] = fmaf(-l4.w, xj, x[3]);
                };
                static_for<15>(sweep);
                const float bcol = X.beta[col];
                __bf16 *dt = reinterpret_cast<__bf16 *>(&Sl.dt[0]);
#pragma unroll
                for (int r = 0; r < 4; ++r) dt[((col >> 2) * 16 + 4 * q + r) * 4 + (col & 3)] = static_cast<__bf16>(x[r] * bcol);
            }
            lds_arrive(&s.ready[pw], lane);
            // this producer's next chunk (past the end: the last chunk again, unused)
            fetch_kq(min(n + 4, nchunks - 1));
            fetch_rest(min(n + 4, nchunks - 1));
        }
    }
}

}  // namespace

bool kda_chunked_supported(const DeltaArgs &a) {
    return a.variant == kKimiDelta && a.dtype == kBF16 && (a.dk == 64 || a.dk == 128) && a.dv % 16 == 0;
}

template <int NVT>
static hipError_t launch_nvt(const DeltaArgs &a, hipStream_t stream) {
    const unsigned blocks = static_cast<unsigned>(a.B * a.H * (a.dv / KdaShape<NVT>::BV));
    switch (a.dk) {
        case 64: kda_chunked_kernel<64, NVT><<<blocks, KdaShape<NVT>::NT, 0, stream>>>(a); break;
        case 128: kda_chunked_kernel<128, NVT><<<blocks, KdaShape<NVT>::NT, 0, stream>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
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
