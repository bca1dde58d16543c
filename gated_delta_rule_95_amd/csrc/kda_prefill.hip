// KDA chunked prefill for gfx950 (MI355X).
//
// Method.  The token recurrence of the Kimi K3 architecture walkthrough
// (mhpq.cn/news/56770, "KDA 到底在算什么": S_t = (I - b k k^T) Diag(a) S_{t-1}
// + b k v^T, o_t = S_t^T q_t, decay -> erase -> write) is evaluated 16 tokens
// at a time.  16 is the decay tile of the pages: with the gate bounded below
// by -5, the cumulative log-decay of 16 tokens stays inside (-80, 0], so the
// rescale factors e^{+-Gc} of a tile are finite in bf16 and fp32 and every
// intra-tile product can be a dense matrix product (K3-on-TPU essay,
// blog.higcp.com, "KDA + Gated MLA", lower-bounded decay; the same section
// of the K3 walkthrough).  For a chunk with entry state S and, per key
// channel, the inclusive cumulative log-decay Gc_r from the chunk start:
//
//   A  = strict_lower(Diag(beta) Kt Kh^T)   Kt = k e^{Gc}, Kh = k e^{-Gc}
//   T  = (I + A)^{-1} Diag(beta)            (unit lower-triangular inverse)
//   X  = V - Kt S,   U = T X
//   O  = Qt S + P U, P = lower_incl(Qt Kh^T), Qt = q e^{Gc}
//   S <- Diag(e^{Gc_16}) S + Kd^T U,        Kd = k e^{Gc_16 - Gc}
//
// which is the token recurrence rearranged (derived from it; the pages only
// sketch the chunked form).
//
// Mapping.  One workgroup per (sequence, head, block of BV = 16 NW columns
// of the state).  The columns of S evolve independently, so the d_v split
// needs no communication.  The workgroup has NW consumer waves and one
// helper wave:
//  * consumer wave w keeps S[:, 16w : 16w+16] of its block in registers, in
//    the 16x16 MFMA accumulator layout (lane l holds rows 4(l/16)+i,
//    column l%16 of each 16x16 tile), and runs the S-dependent chain of
//    chunk c;
//  * the consumer waves together also build the decay-scaled operands of
//    chunk c+2 (cumulative sums, exponentials, bf16 hi/lo splits) into LDS
//    from registers loaded one chunk earlier;
//  * the helper wave forms A and P of chunk c+1 on the matrix cores and
//    inverts (I + A) by forward substitution in fp32.
// Operands live in a three-deep LDS ring; one workgroup barrier per chunk.
//
// Precision.  bf16 inputs: matrix-core operands are bf16 with fp32
// accumulation; the state stays fp32 in registers.  Operands whose rounding
// shows up in o or S (S itself, Qt, T, X, U, P, the Kh behind P, and Kd) are
// kept as bf16 hi + lo pairs; only -Kt (in X and A) is a single bf16; a pair-by-pair product (h1 + l1)(h2 + l2)
// is two 16x16x32 MFMAs whose K slots hold [h1 | l1] against [h2 | h2] and
// [l2 | l2], leaving a relative error near 2^-16 in those terms.  Only the
// 16x16x32 bf16 and 16x16x4 fp32 matrix instructions are used.  fp32 inputs run the same
// schedule on the fp32 matrix cores (v_mfma_f32_16x16x4_f32).
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// ---------------------------------------------------------------------------
// matrix-core wrappers (16x16 output tiles, wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b)
{
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 ld4b(const bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ __forceinline__ bf16x8 ld8b(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ bf16x4 to_bf4(f32x4 x)
{
    return bf16x4{f2bf(x[0]), f2bf(x[1]), f2bf(x[2]), f2bf(x[3])};
}
__device__ __forceinline__ f32x4 from_bf4(bf16x4 x)
{
    return f32x4{bf2f(x[0]), bf2f(x[1]), bf2f(x[2]), bf2f(x[3])};
}

// ---------------------------------------------------------------------------
// configuration
// ---------------------------------------------------------------------------
template <typename TI, int DK_, int NW_>
struct Cfg {
    static constexpr bool BF = std::is_same<TI, bf16>::value;
    using OT = typename std::conditional<BF, bf16, float>::type;   // LDS operand type
    static constexpr int DK = DK_;
    static constexpr int NW = NW_;                 // consumer waves
    static constexpr int BV = 16 * NW;             // state columns per workgroup
    static constexpr int NT = (NW + 1) * WAVE;     // + one helper wave
    static constexpr int NC = NW * WAVE;           // consumer threads
    static constexpr int LDK = DK + (BF ? 8 : 4);  // row stride of [16][DK] arrays
    static constexpr int LDT = BF ? 24 : 20;       // row stride of [*][16] arrays
    static constexpr int LDV = BV + (BF ? 8 : 4);
    static constexpr int LDO = BV + 4;
    // builder: wave w owns CW key channels; lane = (channel pair, token group)
    static constexpr int CW = DK / NW;
    static constexpr int CPW = CW / 2;
    static constexpr int NG = WAVE / CPW;
    static constexpr int TPG = 16 / NG;
    static constexpr int LO = BF ? 1 : 0;          // hi/lo split present
    static_assert(CW >= 16 && CW <= 128, "builder mapping needs 16 <= d_k/NW <= 128");
    static_assert(NG * TPG == 16, "token groups");
};

template <class C>
struct Buf {
    using OT = typename C::OT;
    OT NL[16][C::LDK];                   // -Kt (single precision operand)
    OT QH[16][C::LDK];                   // Qt hi
    OT QL[C::LO ? 16 : 1][C::LDK];       // Qt lo
    OT RH[16][C::LDK];                   // Kh hi
    OT RL[C::LO ? 16 : 1][C::LDK];       // Kh lo
    OT KH[C::DK][C::LDT];                // Kd^T hi   [channel][token]
    OT KL[C::LO ? C::DK : 1][C::LDT];    // Kd^T lo
    OT TH[16][C::LDT];                   // T hi      [token r][token i]
    OT TL[C::LO ? 16 : 1][C::LDT];
    OT PH[16][C::LDT];                   // P hi
    OT PL[C::LO ? 16 : 1][C::LDT];
    OT V[16][C::LDV];                    // value block
    float DEC[C::DK];                    // e^{Gc_16} per channel
    float BETA[16];
};

template <class C>
struct Smem {
    Buf<C> buf[3];
    float AF[16][17];                    // helper: A in fp32
    float OB[2][16][C::LDO];             // output staging
};

// raw (un-scaled) chunk inputs held in registers between load and build
template <class C>
struct Raw {
    using TI = typename std::conditional<C::BF, bf16, float>::type;
    typedef TI TI2 __attribute__((ext_vector_type(2)));
    TI2 q[C::TPG], k[C::TPG];
    f32x2 g[C::TPG];
    typedef TI TI4 __attribute__((ext_vector_type(4)));
    TI4 v;
    float beta;
};

// ---------------------------------------------------------------------------
// loads of one chunk's raw inputs (masked past the sequence end: the padded
// tokens have k = q = v = 0, g = 0, beta = 0, an exact identity transition)
// ---------------------------------------------------------------------------
template <class C, typename TI>
__device__ __forceinline__ void load_raw(Raw<C> &r, const TI *__restrict__ q,
                                         const TI *__restrict__ k, const TI *__restrict__ v,
                                         const float *__restrict__ g,
                                         const float *__restrict__ beta, int64_t tok_base,
                                         int ntok, int H, int h, int DV, int col_base,
                                         int wave, int lane, int tid)
{
    using R = Raw<C>;
    const int cp = lane % C::CPW, tg = lane / C::CPW;
    const int ch = wave * C::CW + 2 * cp;
#pragma unroll
    for (int t = 0; t < C::TPG; ++t) {
        const int tok = tg * C::TPG + t;
        if (tok < ntok) {
            const int64_t e = ((tok_base + tok) * H + h) * (int64_t)C::DK + ch;
            r.q[t] = *reinterpret_cast<const typename R::TI2 *>(q + e);
            r.k[t] = *reinterpret_cast<const typename R::TI2 *>(k + e);
            r.g[t] = *reinterpret_cast<const f32x2 *>(g + e);
        } else {
            r.q[t] = typename R::TI2{(TI)0.f, (TI)0.f};
            r.k[t] = typename R::TI2{(TI)0.f, (TI)0.f};
            r.g[t] = f32x2{0.f, 0.f};
        }
    }
    {
        const int row = tid / (C::BV / 4), c4 = tid % (C::BV / 4);
        if (row < ntok) {
            const int64_t e = ((tok_base + row) * H + h) * (int64_t)DV + col_base + 4 * c4;
            r.v = *reinterpret_cast<const typename R::TI4 *>(v + e);
        } else {
            r.v = typename R::TI4{(TI)0.f, (TI)0.f, (TI)0.f, (TI)0.f};
        }
    }
    r.beta = (tid < ntok) ? beta[(tok_base + tid) * H + h] : 0.f;
}

// ---------------------------------------------------------------------------
// build: raw registers -> decay-scaled operands of one chunk in LDS
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void store_pair(typename C::OT *hi, typename C::OT *lo, float a, float b)
{
    using OT = typename C::OT;
    typedef OT OT2 __attribute__((ext_vector_type(2)));
    if constexpr (C::BF) {
        const bf16 ah = f2bf(a), bh = f2bf(b);
        *reinterpret_cast<OT2 *>(hi) = OT2{ah, bh};
        *reinterpret_cast<OT2 *>(lo) = OT2{f2bf(a - bf2f(ah)), f2bf(b - bf2f(bh))};
    } else {
        *reinterpret_cast<OT2 *>(hi) = OT2{a, b};
    }
}

template <class C>
__device__ __forceinline__ void build(Buf<C> &B, const Raw<C> &r, int wave, int lane, int tid)
{
    using OT = typename C::OT;
    typedef OT OT2 __attribute__((ext_vector_type(2)));
    const int cp = lane % C::CPW, tg = lane / C::CPW;
    const int ch = wave * C::CW + 2 * cp;

    // cumulative log2-decay over this lane's tokens, then across token groups
    float G0[C::TPG], G1[C::TPG];
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int t = 0; t < C::TPG; ++t) {
        s0 += r.g[t][0] * LOG2E;
        s1 += r.g[t][1] * LOG2E;
        G0[t] = s0;
        G1[t] = s1;
    }
    float i0 = s0, i1 = s1;     // inclusive scan of group totals
#pragma unroll
    for (int off = 1; off < C::NG; off <<= 1) {
        const float n0 = __shfl_up(i0, off * C::CPW, WAVE);
        const float n1 = __shfl_up(i1, off * C::CPW, WAVE);
        if (tg >= off) { i0 += n0; i1 += n1; }
    }
    const float e0 = i0 - s0, e1 = i1 - s1;                  // exclusive offsets
    const int last = cp + (C::NG - 1) * C::CPW;
    const float T0 = __shfl(i0, last, WAVE), T1 = __shfl(i1, last, WAVE);  // Gc_16
    const float inv0 = fast_exp2(-T0), inv1 = fast_exp2(-T1);

#pragma unroll
    for (int t = 0; t < C::TPG; ++t) {
        const int tok = tg * C::TPG + t;
        const float ga = G0[t] + e0, gb = G1[t] + e1;
        const float pa = fast_exp2(ga), pb = fast_exp2(gb);           // e^{Gc}
        const float sa = fast_exp2(T0 - ga), sb = fast_exp2(T1 - gb); // e^{Gc_16 - Gc}
        const float ka = (float)r.k[t][0], kb = (float)r.k[t][1];
        const float qa = (float)r.q[t][0], qb = (float)r.q[t][1];
        *reinterpret_cast<OT2 *>(&B.NL[tok][ch]) = OT2{(OT)(-ka * pa), (OT)(-kb * pb)};
        store_pair<C>(&B.QH[tok][ch], &B.QL[C::LO ? tok : 0][ch], qa * pa, qb * pb);
        const float da = ka * sa, db = kb * sb;                       // Kd
        store_pair<C>(&B.RH[tok][ch], &B.RL[C::LO ? tok : 0][ch], da * inv0, db * inv1);
        // Kd^T: [channel][token]
        if constexpr (C::BF) {
            const bf16 ha = f2bf(da), hb = f2bf(db);
            B.KH[ch][tok] = ha;
            B.KH[ch + 1][tok] = hb;
            B.KL[ch][tok] = f2bf(da - bf2f(ha));
            B.KL[ch + 1][tok] = f2bf(db - bf2f(hb));
        } else {
            B.KH[ch][tok] = da;
            B.KH[ch + 1][tok] = db;
        }
    }
    if (tg == 0) {
        B.DEC[ch] = fast_exp2(T0);
        B.DEC[ch + 1] = fast_exp2(T1);
    }
    {
        const int row = tid / (C::BV / 4), c4 = tid % (C::BV / 4);
        typedef OT OT4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<OT4 *>(&B.V[row][4 * c4]) =
            OT4{(OT)(float)r.v[0], (OT)(float)r.v[1], (OT)(float)r.v[2], (OT)(float)r.v[3]};
    }
    if (tid < 16) B.BETA[tid] = r.beta;
}

// ---------------------------------------------------------------------------
// helper wave: A, P and T = (I + A)^{-1} Diag(beta) for one chunk
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void helper(Buf<C> &B, float (*AF)[17], int lane)
{
    const int j = lane & 15, g4 = lane >> 4;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
    if constexpr (C::BF) {
        if constexpr (C::DK >= 32) {
            // K slot (g4, i) = channel 32 s + 8 g4 + i on both operands
#pragma unroll
            for (int s = 0; s < C::DK / 32; ++s) {
                const int kk = 32 * s + 8 * g4;
                const bf16x8 nl = ld8b(&B.NL[j][kk]);
                const bf16x8 qh = ld8b(&B.QH[j][kk]), ql = ld8b(&B.QL[j][kk]);
                const bf16x8 rh = ld8b(&B.RH[j][kk]), rl = ld8b(&B.RL[j][kk]);
                a = mma32(nl, rh, a);
                p = mma32(qh, rh, p);
                p = mma32(qh, rl, p);
                p = mma32(ql, rh, p);
            }
        } else {
            // d_k = 16: K slot (g4, i) = channel 4 g4 + i%4 of the hi (i < 4)
            // or lo (i >= 4) part
            const int kk = 4 * g4;
            const bf16x4 nl = ld4b(&B.NL[j][kk]);
            const bf16x4 qh = ld4b(&B.QH[j][kk]), ql = ld4b(&B.QL[j][kk]);
            const bf16x4 rh = ld4b(&B.RH[j][kk]), rl = ld4b(&B.RL[j][kk]);
            const bf16x4 z = {};
            a = mma32(cat(nl, z), cat(rh, z), a);
            p = mma32(cat(qh, ql), cat(rh, rh), p);      // (qh + ql) rh
            p = mma32(cat(qh, ql), cat(rl, rl), p);      // (qh + ql) rl
        }
    } else {
#pragma unroll 8
        for (int s = 0; s < C::DK / 4; ++s) {
            const int kk = 4 * s + g4;
            a = mma4(B.NL[j][kk], B.RH[j][kk], a);
            p = mma4(B.QH[j][kk], B.RH[j][kk], p);
        }
    }
    // D layout: element i of lane (j, g4) is row r = 4 g4 + i, column j.
    // A_{ri} = beta_r Kt_r . Kh_i for i < r; NL = -Kt, hence the sign.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        AF[r][j] = (j < r) ? -B.BETA[r] * a[i] : 0.f;
        const float pv = (j <= r) ? p[i] : 0.f;
        if constexpr (C::BF) {
            const bf16 ph = f2bf(pv);
            B.PH[r][j] = ph;
            B.PL[r][j] = f2bf(pv - bf2f(ph));
        } else {
            B.PH[r][j] = pv;
        }
    }
    // make this wave's AF writes visible to its own later reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < 16) {
        // column j of (I + A)^{-1}: forward substitution, fp32
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= AF[r][i] * t[i];
            t[r] = acc;
        }
        const float bj = B.BETA[j];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float tv = t[r] * bj;
            if constexpr (C::BF) {
                const bf16 th = f2bf(tv);
                B.TH[r][j] = th;
                B.TL[r][j] = f2bf(tv - bf2f(th));
            } else {
                B.TH[r][j] = tv;
            }
        }
    }
}

// hi/lo bf16 split of a D-layout tile, packed as 32-deep B operands:
// hh = [hi; hi], ll = [lo; lo] (slot (g4, i) = row 4 g4 + i%4)
__device__ __forceinline__ void split_hl(f32x4 x, bf16x8 &hh, bf16x8 &ll)
{
    const bf16x4 h = to_bf4(x);
    const bf16x4 l = to_bf4(x - from_bf4(h));
    hh = cat(h, h);
    ll = cat(l, l);
}

// ---------------------------------------------------------------------------
// consumer wave: the S-dependent chain of one chunk
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void consume(const Buf<C> &B, f32x4 (&S)[C::DK / 16],
                                        float (*OB)[C::LDO], int wave, int lane)
{
    const int j = lane & 15, g4 = lane >> 4;
    const int vc = 16 * wave + j;           // column inside the block
    f32x4 x, u, o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)B.V[4 * g4 + i][vc];

    if constexpr (C::BF) {
        // S as a bf16 hi/lo pair of B operands.  For d_k >= 32 the K slot
        // (g4, i) of step s is channel 32 s + 4 g4 + i (i < 4, tile 2s) or
        // 32 s + 16 + 4 g4 + (i - 4) (tile 2s + 1); A operands are read with
        // the same assignment, so each product is an exact contraction.
        if constexpr (C::DK >= 32) {
            constexpr int NS = C::DK / 32;
            bf16x8 sh[NS], sl[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bf16x4 h0 = to_bf4(S[2 * s]), h1 = to_bf4(S[2 * s + 1]);
                sh[s] = cat(h0, h1);
                sl[s] = cat(to_bf4(S[2 * s] - from_bf4(h0)), to_bf4(S[2 * s + 1] - from_bf4(h1)));
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int kk = 32 * s + 4 * g4;
                const bf16x8 nl = cat(ld4b(&B.NL[j][kk]), ld4b(&B.NL[j][kk + 16]));
                const bf16x8 qh = cat(ld4b(&B.QH[j][kk]), ld4b(&B.QH[j][kk + 16]));
                const bf16x8 ql = cat(ld4b(&B.QL[j][kk]), ld4b(&B.QL[j][kk + 16]));
                x = mma32(nl, sh[s], x);
                x = mma32(nl, sl[s], x);
                o = mma32(qh, sh[s], o);            // Qt S: the lo x lo term
                o = mma32(qh, sl[s], o);            // (2^-18) is dropped
                o = mma32(ql, sh[s], o);
            }
        } else {
            // d_k = 16: slot (g4, i) = channel 4 g4 + i%4 of S hi (i < 4) or lo
            const bf16x4 h = to_bf4(S[0]);
            const bf16x8 shl = cat(h, to_bf4(S[0] - from_bf4(h)));
            const bf16x4 nl = ld4b(&B.NL[j][4 * g4]);
            const bf16x8 qq = cat(ld4b(&B.QH[j][4 * g4]), ld4b(&B.QL[j][4 * g4]));
            x = mma32(cat(nl, nl), shl, x);
            o = mma32(qq, cat(h, h), o);                     // (Qh + Ql) Sh
            o = mma32(qq, cat(shl.hi, shl.hi), o);           // (Qh + Ql) Sl
        }
        // U = T X with both as hi/lo pairs: (Th + Tl)(Xh + Xl)
        bf16x8 xhh, xll, uhh, ull;
        split_hl(x, xhh, xll);
        const bf16x8 t = cat(ld4b(&B.TH[j][4 * g4]), ld4b(&B.TL[j][4 * g4]));
        u = mma32(t, xhh, f32x4{0.f, 0.f, 0.f, 0.f});
        u = mma32(t, xll, u);
        split_hl(u, uhh, ull);
        // O += P U
        const bf16x8 pp = cat(ld4b(&B.PH[j][4 * g4]), ld4b(&B.PL[j][4 * g4]));
        o = mma32(pp, uhh, o);
        o = mma32(pp, ull, o);
        // S <- Diag(e^{Gc_16}) S + Kd^T U
#pragma unroll
        for (int t4 = 0; t4 < C::DK / 16; ++t4) {
            const f32x4 dec = *reinterpret_cast<const f32x4 *>(&B.DEC[16 * t4 + 4 * g4]);
            const bf16x8 kd = cat(ld4b(&B.KH[16 * t4 + j][4 * g4]),
                                  ld4b(&B.KL[16 * t4 + j][4 * g4]));
            S[t4] *= dec;
            S[t4] = mma32(kd, uhh, S[t4]);
            S[t4] = mma32(kd, ull, S[t4]);
        }
    } else {
        // fp32: K index of slot (g4) in step (t, i) is 16 t + 4 g4 + i
#pragma unroll
        for (int t = 0; t < C::DK / 16; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 16 * t + 4 * g4 + i;
                x = mma4(B.NL[j][kk], S[t][i], x);
                o = mma4(B.QH[j][kk], S[t][i], o);
            }
        }
        u = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) u = mma4(B.TH[j][4 * g4 + i], x[i], u);
#pragma unroll
        for (int i = 0; i < 4; ++i) o = mma4(B.PH[j][4 * g4 + i], u[i], o);
#pragma unroll
        for (int t = 0; t < C::DK / 16; ++t) {
            const f32x4 dec = *reinterpret_cast<const f32x4 *>(&B.DEC[16 * t + 4 * g4]);
            S[t] *= dec;
#pragma unroll
            for (int i = 0; i < 4; ++i) S[t] = mma4(B.KH[16 * t + j][4 * g4 + i], u[i], S[t]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) OB[4 * g4 + i][vc] = o[i];
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <typename TI, typename TO, int DK, int DV, int NW>
__global__ __launch_bounds__((Cfg<TI, DK, NW>::NT))
void kda_prefill_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                        const TI *__restrict__ v, const float *__restrict__ g,
                        const float *__restrict__ beta, const float *__restrict__ S0,
                        const int32_t *__restrict__ cu_seqlens, int32_t seqlen,
                        int32_t n_chains, int32_t H, TO *__restrict__ o,
                        float *__restrict__ S_T)
{
    using C = Cfg<TI, DK, NW>;
    constexpr int NB = DV / C::BV;
    __shared__ Smem<C> sm;

    // workgroup -> (chain, column block); the NB blocks of a chain share an
    // XCD (workgroups are dealt round-robin over the 8 XCDs), so the chain's
    // q/k/g are fetched from HBM once and re-read from that XCD's L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, rest = bid >> 3;
    const int vb = rest % NB;
    const int chain = (rest / NB) * 8 + xcd;
    if (chain >= n_chains) return;
    const int n = chain / H, h = chain % H;
    int64_t bos, T;
    if (cu_seqlens) {
        bos = cu_seqlens[n];
        T = (int64_t)cu_seqlens[n + 1] - bos;
        if (T < 0) T = 0;
    } else {
        bos = (int64_t)n * seqlen;
        T = seqlen;
    }
    const int nch = (int)((T + 15) / 16);
    const int col_base = vb * C::BV;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool is_helper = wave == NW;
    const int j = lane & 15, g4 = lane >> 4;

    // consumer state: S[:, col_base + 16 wave + j], rows 16 t + 4 g4 + i
    f32x4 S[DK / 16];
    const int64_t sbase = (int64_t)chain * DK * DV + col_base + 16 * wave + j;
    if (!is_helper) {
#pragma unroll
        for (int t = 0; t < DK / 16; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[t][i] = S0 ? S0[sbase + (int64_t)(16 * t + 4 * g4 + i) * DV] : 0.f;
    }

    Raw<C> raw;
    if (!is_helper && nch > 0)
        load_raw<C>(raw, q, k, v, g, beta, bos, (int)(T < 16 ? T : 16), H, h, DV, col_base,
                    wave, lane, tid);

    for (int c = -2; c < nch; ++c) {
        if (!is_helper) {
            const int cb = c + 2;             // chunk to build
            if (cb < nch) {
                build<C>(sm.buf[cb % 3], raw, wave, lane, tid);
                const int cl = c + 3;         // chunk to load
                if (cl < nch) {
                    const int64_t rem = T - 16 * (int64_t)cl;
                    load_raw<C>(raw, q, k, v, g, beta, bos + 16 * (int64_t)cl,
                                (int)(rem < 16 ? rem : 16), H, h, DV, col_base, wave, lane, tid);
                }
            }
            if (c >= 1) {                     // write out chunk c - 1
                const int cs = c - 1;
                const int64_t rem = T - 16 * (int64_t)cs;
                const int row = tid / (C::BV / 4), c4 = tid % (C::BV / 4);
                if (row < rem) {
                    const float *src = &sm.OB[cs & 1][row][4 * c4];
                    const int64_t e = ((bos + 16 * (int64_t)cs + row) * H + h) * (int64_t)DV +
                                      col_base + 4 * c4;
                    Elem<TO>::st4(o + e, f32x4{src[0], src[1], src[2], src[3]});
                }
            }
            if (c >= 0) consume<C>(sm.buf[c % 3], S, sm.OB[c & 1], wave, lane);
        } else {
            const int ch = c + 1;
            if (ch >= 0 && ch < nch) helper<C>(sm.buf[ch % 3], sm.AF, lane);
        }
        __syncthreads();
    }
    if (!is_helper) {
        if (nch >= 1) {
            const int cs = nch - 1;
            const int64_t rem = T - 16 * (int64_t)cs;
            const int row = tid / (C::BV / 4), c4 = tid % (C::BV / 4);
            if (row < rem) {
                const float *src = &sm.OB[cs & 1][row][4 * c4];
                const int64_t e = ((bos + 16 * (int64_t)cs + row) * H + h) * (int64_t)DV +
                                  col_base + 4 * c4;
                Elem<TO>::st4(o + e, f32x4{src[0], src[1], src[2], src[3]});
            }
        }
        if (S_T) {
#pragma unroll
            for (int t = 0; t < DK / 16; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S_T[sbase + (int64_t)(16 * t + 4 * g4 + i) * DV] = S[t][i];
        }
    }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
template <typename TI, typename TO, int DK, int DV, int NW>
static hipError_t launch_t(const PrefillArgs &a)
{
    using C = Cfg<TI, DK, NW>;
    static_assert(DV % C::BV == 0, "column blocks");
    constexpr int NB = DV / C::BV;
    const int64_t chains = (int64_t)a.n_seqs * a.H;
    if (chains == 0) return hipSuccess;
    if (chains > INT32_MAX - 8) return hipErrorInvalidValue;
    const int64_t grid = ((chains + 7) / 8) * 8 * NB;
    if (grid * C::NT >= ((int64_t)1 << 32)) return hipErrorInvalidValue;  // grid size limit
    hipLaunchKernelGGL((kda_prefill_kernel<TI, TO, DK, DV, NW>), dim3((unsigned)grid),
                       dim3(C::NT), 0, (hipStream_t)a.stream, (const TI *)a.q,
                       (const TI *)a.k, (const TI *)a.v, a.g, a.beta, a.S0, a.cu_seqlens,
                       a.seqlen, (int32_t)chains, a.H, (TO *)a.o, a.S_T);
    return hipGetLastError();
}

// waves per workgroup: 16 columns per consumer wave, at most 4 consumers
template <int DK, int DV>
struct PickNW {
    static constexpr int byv = DV / 16 < 4 ? DV / 16 : 4;
    static constexpr int bydk = DK / 16;                 // builder needs d_k/NW >= 16
    static constexpr int value = byv < bydk ? byv : bydk;
};

template <typename TI, typename TO>
static hipError_t dispatch_dims(const PrefillArgs &a)
{
#define KDA_PF_CASE(DK_, DV_) \
    if (a.d_k == DK_ && a.d_v == DV_) return launch_t<TI, TO, DK_, DV_, PickNW<DK_, DV_>::value>(a);
    KDA_PF_CASE(16, 16) KDA_PF_CASE(16, 32) KDA_PF_CASE(16, 64) KDA_PF_CASE(16, 128)
    KDA_PF_CASE(32, 16) KDA_PF_CASE(32, 32) KDA_PF_CASE(32, 64) KDA_PF_CASE(32, 128)
    KDA_PF_CASE(64, 16) KDA_PF_CASE(64, 32) KDA_PF_CASE(64, 64) KDA_PF_CASE(64, 128)
    KDA_PF_CASE(128, 16) KDA_PF_CASE(128, 32) KDA_PF_CASE(128, 64) KDA_PF_CASE(128, 128)
#undef KDA_PF_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs &a)
{
    if (a.in_bf16) {
        return a.out_bf16 ? dispatch_dims<bf16, bf16>(a) : dispatch_dims<bf16, float>(a);
    }
    return dispatch_dims<float, float>(a);
}

}  // namespace kda
