// KDA chunked prefill for gfx950 (MI355X).
//
// Method.  The token recurrence of the Kimi K3 architecture walkthrough
// (mhpq.cn/news/56770, "KDA 到底在算什么": S_t = (I - b k k^T) Diag(a) S_{t-1}
// + b k v^T, o_t = S_t^T q_t, decay -> erase -> write) is evaluated 16 tokens
// at a time.  16 is the decay tile of the pages: with the gate bounded below
// by -5, the cumulative log-decay of 16 tokens stays inside (-80, 0], so the
// rescale factors of a tile are finite in bf16 and fp32 and every intra-tile
// product can be a dense matrix product (K3-on-TPU essay, blog.higcp.com,
// "KDA + Gated MLA", lower-bounded decay; the lower-bounded-decay section of
// the K3 walkthrough).
//
// Chunk algebra (derived from the recurrence; the pages only sketch the
// chunked form).  For a chunk of 16 tokens with entry state S and, per key
// channel, the inclusive cumulative log-decay Gc_r from the chunk start, let
// Gc_16 be the chunk total and reference every factor to the chunk END:
//
//   E_r  = e^{Gc_r - Gc_16}  in [1, e^75]      Kd_r = k_r e^{Gc_16 - Gc_r}  (<= |k_r|)
//   KE_r = k_r E_r,  QE_r = q_r E_r,            Sd = Diag(e^{Gc_16}) S   (the decayed state)
//
//   A  = strict_lower(Diag(beta) KE Kd^T),      P = lower_incl(QE Kd^T)
//   T  = (I + A)^{-1} Diag(beta)                (unit lower-triangular inverse)
//   X  = V - KE Sd,    U = T X
//   O  = QE Sd + P U
//   S' = Sd + Kd^T U
//
// since k_r e^{Gc_r} S = KE_r Sd and (k_r e^{Gc_r}).(k_i e^{-Gc_i}) = KE_r.Kd_i.
// A term lost to underflow of Sd is below FLT_MIN e^75 (~4e-6) in absolute
// value.
//
// Mapping.  One workgroup per (sequence, head, block of BV = 16 NW columns
// of the state): the columns of S evolve independently, so the d_v split
// needs no communication.  Three roles, NW + NBW + 2 waves:
//  * consumer wave w keeps S[:, 16w : 16w+16] of its block in registers in
//    the 16x16 MFMA accumulator layout (lane l holds rows 4(l/16)+i, column
//    l%16 of each 16x16 tile) and runs the S-dependent chain of chunk c;
//  * builder wave w loads the raw inputs of 1/NBW of the key channels (and
//    of the value block) and builds the operands of chunk c+2 (cumulative
//    sums, exponentials, bf16 hi/lo splits) into LDS;
//  * two helper waves, on different SIMDs, form A of chunk c+1 and the
//    inverse of (I + A) as a product of four factors, and P of chunk c+1,
//    all on the matrix cores.
// A ring of three LDS operand slots needs one barrier per chunk.
//
// Precision.  bf16 inputs: matrix-core operands are bf16 with fp32
// accumulation; the state stays fp32 in registers.  Operands whose rounding
// shows up in o or S (Sd, QE, T, X, U, P and Kd) are bf16 hi + lo pairs; a
// pair-by-pair product (h1 + l1)(h2 + l2) is two 16x16x32 MFMAs whose K slots
// hold [h1 | l1] against [h2 | h2] and [l2 | l2], or [h1 | h1] and [l1 | l1]
// against [h2 | l2] (three for QE Sd, where the K slots are all channels),
// leaving a relative error near 2^-16.  Only -KE
// (in X and A) is a single bf16.  fp32 inputs run the same schedule on the
// fp32 matrix cores (v_mfma_f32_16x16x4_f32).
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>
#include <vector>

#include "kda_chunk.h"
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {


// ---------------------------------------------------------------------------
// Operands of a chunk that its builders have already finished (v block, the
// decay of the first two state tiles, the first 32-deep step of -KE and QE).
// The consumer reads them for chunk c + 1 before the barrier that ends chunk
// c, so the next chain starts without waiting on LDS.  T and P, which the
// helper writes during chunk c, are not among them.
// ---------------------------------------------------------------------------
template <class C>
struct Ahead {
    using OT = typename C::OT;
    typedef OT OT4 __attribute__((ext_vector_type(4)));
    OT4 v;
    f32x4 dec[C::DK >= 32 ? 2 : 1];
    bf16x8 nk, qh, ql;                   // bf16 with d_k >= 32 only
};
template <class C>
__device__ __forceinline__ void read_ahead(const Buf<C> &B, Ahead<C> &a, int wave, int lane)
{
    typedef typename Ahead<C>::OT4 OT4;
    const int j = lane & 15, g4 = lane >> 4;
    a.v = *reinterpret_cast<const OT4 *>(&B.VT[16 * wave + j][4 * g4]);
#pragma unroll
    for (int t = 0; t < (C::DK >= 32 ? 2 : 1); ++t)
        a.dec[t] = *reinterpret_cast<const f32x4 *>(&B.DEC[16 * t + 4 * g4]);
    if constexpr (C::BF && C::DK >= 32) {
        a.nk = ld8b(&B.NK[j][8 * g4]);
        a.qh = ld8b(&B.QH[j][8 * g4]);
        a.ql = ld8b(&B.QL[j][8 * g4]);
    }
}

// ---------------------------------------------------------------------------
// consumer wave: the S-dependent chain of one chunk; returns O transposed in
// the D layout: lane (j, g4) holds O[token j][columns 4 g4 .. 4 g4 + 3].
// With CKS (the checkpointing forward, bf16, d_k >= 32) it also stores the
// chunk's Sd hi/lo operands, 16 bytes per lane each, at cks[(2 s + {0, 1}) x
// 64 lanes]: the backward's chunk kernel takes them as they are.
// ---------------------------------------------------------------------------
template <class C, bool CKS = false>
__device__ __forceinline__ f32x4 consume(const Buf<C> &B, f32x4 (&S)[C::DK / 16],
                                         const Ahead<C> &ah, int wave, int lane,
                                         u32x4 *cks = nullptr)
{
    const int j = lane & 15, g4 = lane >> 4;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const NegEye ne = neg_eye(lane);
    f32x4 x, u, o = zero;
    // X = V - KE Sd; gated, the product is scaled by s_k per token first
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = C::GATED ? 0.f : (float)ah.v[i];
    // Sd = Diag(e^{Gc_16}) S
#pragma unroll
    for (int t = 0; t < C::DK / 16; ++t)
        S[t] *= t < (C::DK >= 32 ? 2 : 1) ? ah.dec[t < 1 ? 0 : C::DK >= 32 ? 1 : 0]
                                          : *reinterpret_cast<const f32x4 *>(&B.DEC[16 * t + 4 * g4]);

    if constexpr (C::BF) {
        // T and P of the chunk are final when the chunk starts: read first
        const bf16x8 th2 = ld8b(&B.TH[j][8 * g4]), tl2 = ld8b(&B.TL[j][8 * g4]);
        const bf16x8 ph2 = ld8b(&B.PH[j][8 * g4]), pl2 = ld8b(&B.PL[j][8 * g4]);
        bf16x8 kd[C::DK / 16];
        auto load_kd = [&]() {
#pragma unroll
            for (int t = 0; t < C::DK / 16; ++t) kd[t] = ld8b(&B.KH[16 * t + j][8 * g4]);
        };
        // Sd as a bf16 hi/lo pair of B operands.  For d_k >= 32 the K slot
        // (g4, i) of step s is channel 32 s + 4 g4 + i (i < 4, tile 2s) or
        // 32 s + 16 + 4 g4 + (i - 4) (tile 2s + 1); A operands are read with
        // the same assignment, so each product is an exact contraction.
        if constexpr (C::DK >= 32) {
            constexpr int NS = C::DK / 32;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (s == NS - 1) {
                    // the state-update operands are issued here (the earlier
                    // steps' operand registers are free again), so they
                    // arrive while the last step and the U chain run; the
                    // scheduling barrier keeps the compiler from sinking them
                    load_kd();
                    __builtin_amdgcn_sched_barrier(0);
                }
                bf16x8 sh, sl;
                split8(S[2 * s], S[2 * s + 1], ne, sh, sl);
                if constexpr (CKS) {          // read once, by the backward: streamed
                    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sh), &cks[(2 * s) * WAVE]);
                    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sl), &cks[(2 * s + 1) * WAVE]);
                }
                // stored positions 32 s + 8 g4 .. + 7 hold exactly these channels
                const int kk = 32 * s + 8 * g4;
                const bf16x8 nk = s == 0 ? ah.nk : ld8b(&B.NK[j][kk]);
                const bf16x8 qh = s == 0 ? ah.qh : ld8b(&B.QH[j][kk]);
                const bf16x8 ql = s == 0 ? ah.ql : ld8b(&B.QL[j][kk]);
                // -KE is a single bf16, so Sd's lo part would add nothing to
                // X beyond KE's own rounding (checked in emulation against the
                // oracle: o and S_T errors unchanged); only Sd hi enters X
                x = mma32(nk, sh, x);
                // O^T = Sd^T QE^T: the state is the A operand, so each lane
                // ends with four consecutive output columns of one token
                o = mma32(sh, qh, o);            // the lo x lo term
                o = mma32(sl, qh, o);            // (2^-18) is dropped
                o = mma32(sh, ql, o);
            }
        } else {
            // d_k = 16: slot (g4, i) = channel 4 g4 + i%4 of Sd hi (i < 4) or lo
            load_kd();
            bf16x4 hh, ll;
            split4(S[0], ne, hh, ll);
            const bf16x4 nk = ld4b(&B.NK[j][4 * g4]);
            const bf16x4 qh = ld4b(&B.QH[j][4 * g4]), ql = ld4b(&B.QL[j][4 * g4]);
            x = mma32(cat(nk, nk), cat(hh, ll), x);
            o = mma32(cat(hh, ll), cat(qh, qh), o);          // (Sh + Sl) Qh
            o = mma32(cat(hh, ll), cat(ql, ql), o);          // (Sh + Sl) Ql
        }
        if constexpr (C::GATED) {
            const f32x4 sk4 = *reinterpret_cast<const f32x4 *>(&B.SK[4 * g4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = __builtin_fmaf(sk4[i], x[i], (float)ah.v[i]);
        }
        // U = T X with both as hi/lo pairs: [Th | Th] and [Tl | Tl] against
        // [Xh; Xl]
        bf16x8 uhh, ull;
        bf16x4 xh, xl;
        split4(x, ne, xh, xl);
        const bf16x8 xhl = cat(xh, xl);
        u = mma32(th2, xhl, zero);
        u = mma32(tl2, xhl, u);
        bf16x4 uh, ul;
        split4(u, ne, uh, ul);
        uhh = cat(uh, uh);
        ull = cat(ul, ul);
        // O^T += U^T P^T: [Uh | Ul] against [Ph | Ph] and [Pl | Pl]
        const bf16x8 uhl = cat(uh, ul);
        o = mma32(uhl, ph2, o);
        o = mma32(uhl, pl2, o);
        // S' = Sd + Kd^T U
#pragma unroll
        for (int t = 0; t < C::DK / 16; ++t) {
            S[t] = mma32(kd[t], uhh, S[t]);
            S[t] = mma32(kd[t], ull, S[t]);
        }
    } else {
        // fp32: K index of slot (g4) in step (t, i) is 16 t + 4 g4 + i
#pragma unroll
        for (int t = 0; t < C::DK / 16; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 16 * t + 4 * g4 + i;
                x = mma4(B.NK[j][kk], S[t][i], x);
                o = mma4(S[t][i], B.QH[j][kk], o);           // O^T
            }
        }
        if constexpr (C::GATED) {
            const f32x4 sk4 = *reinterpret_cast<const f32x4 *>(&B.SK[4 * g4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = __builtin_fmaf(sk4[i], x[i], (float)ah.v[i]);
        }
        u = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) u = mma4(B.TH[j][4 * g4 + i], x[i], u);
#pragma unroll
        for (int i = 0; i < 4; ++i) o = mma4(u[i], B.PH[j][4 * g4 + i], o);
#pragma unroll
        for (int t = 0; t < C::DK / 16; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) S[t] = mma4(B.KH[16 * t + j][4 * g4 + i], u[i], S[t]);
        }
    }
    // gated: O = Diag(s_q) (Q~E Sd + P~ U'), with U' = Diag(s_k) U from T
    if constexpr (C::GATED) o *= B.SQ[j];
    return o;
}

// ---------------------------------------------------------------------------
// Launch parameters.  Every workgroup runs one job: a token range of one
// (sequence, head) chain and one block of BV state columns.
//
// Without a sequence split (nseg == 1) a job is a whole sequence and one
// block of the d_v value columns.
//
// With a split, each sequence's tokens are cut into segment 0 (the first
// len0 tokens) and segments 1 .. nseg-1 (lenS tokens each, the last one
// possibly shorter).  Segment 0 runs from S0 as usual and leaves its final
// state as the entry state of segment 1.  A later segment runs from a zero
// state and carries, next to its d_v value columns, the d_k columns of the
// segment's transition: those start from the identity with zero values, so
// they evolve into M = Phi (the product of the segment's per-token maps
// S -> (I - b k k^T) Diag(alpha) S) and their outputs are R_t = Phi_t^T q_t.
// Then  S_end = M S_entry + S~  and  o_t = o~_t + S_entry^T R_t  for every
// token t of the segment, where S~ and o~ come from the value columns.  The
// scan and the correction kernels below apply these once the entry states
// are known.  (Affine summary of a segment and a prefix scan over segments:
// K3-on-TPU essay, blog.higcp.com, the section on the existing TPU kernel;
// used across compute units of one device, the intra-device sequence-split
// regime of the same essay's "KDA + Gated MLA" costs section, item (3).)
// ---------------------------------------------------------------------------
template <typename TI, typename TO>
struct Params {
    const TI *q, *k, *v;
    const float *g, *beta, *S0;
    const int32_t *cu_seqlens;   // nullptr: equal lengths seqlen
    TO *o;
    float *S_T;
    int32_t seqlen, n_tokens, n_chains, chains8, H;
    // sequence split (nseg == 1: none; only with cu_seqlens == nullptr)
    int32_t nseg, len0, lenS;
    float *sumst;   // [chain][nseg-1][d_k][d_v + d_k]  final states of segments 1..
    float *entry;   // [chain][nseg-1][d_k][d_v]        entry states of segments 1..
    float *o0;      // [n_seqs][seqlen - len0][H][d_v]  zero-start outputs o~
    float *rq;      // [n_seqs][seqlen - len0][H][d_k]  pulled-back queries R
    // gated prologue: z [tokens][H][d_k] and b [tokens][H] in the input
    // type replace g and beta; A_log [H]
    const TI *z, *braw;
    const float *A_log;
    // checkpointing variant (backward support): the state at the start of
    // every chunk c of sequence n goes to slot bos / 16 + n + c of ckpt, 64
    // KiB per slot and head at d = 128; o is not written.  fp32 inputs or
    // d_k = 16: [slot][H][d_v / 16][d_k / 16][64][4] floats, per 16 x 16 tile
    // (key rows 16 t .., value columns 16 cb ..) lane j + 16 g holds rows
    // 16 t + 4 g .. + 3 of column 16 cb + j.  bf16 with d_k >= 32: the
    // decayed state Sd = Diag(e^{Gc_16}) S as the consumer's operands,
    // [slot][H][d_v / 16][d_k / 32][hi, lo][64][16 bytes], lane j + 16 g of
    // step s holding channels 32 s + 4 g .. + 3 and 32 s + 16 + 4 g .. + 3 of
    // column 16 cb + j
    float *ckpt;
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <typename TI, typename TO, int DK, int DV, int NW, int NBUF, bool GATED, bool CKPT>
__global__ __launch_bounds__((Cfg<TI, DK, NW, NBUF, GATED>::NT), 1)
void kda_prefill_kernel(const Params<TI, TO> p)
{
    static_assert(!(CKPT && GATED), "the checkpointing variant takes g and beta");
    using C = Cfg<TI, DK, NW, NBUF, GATED>;
    constexpr int NB = DV / C::BV;               // value column blocks of a chain
    constexpr int NA = NB + DK / C::BV;          // ... plus transition blocks (split)
    constexpr int LAG = NBUF - 1;            // build runs LAG chunks ahead
    __shared__ Smem<C> sm;
    const int H = p.H;

    // Workgroup -> job.  Jobs come in groups, one per segment, longest
    // first (segment 0, then segments 1, 2, ...), each group chains8 x
    // (blocks per chain) workgroups.  Inside a group the blocks of a chain
    // share an XCD (workgroups are dealt round-robin over the 8 XCDs), so
    // the chain's q/k/g are fetched from HBM once and re-read from that
    // XCD's L2.
    int bid = blockIdx.x, seg = 0, W = NB;
    if (bid >= p.chains8 * NB) {
        const int r = bid - p.chains8 * NB;
        seg = 1 + r / (p.chains8 * NA);
        bid = r % (p.chains8 * NA);
        W = NA;
    }
    const int xcd = bid & 7, rest = bid >> 3;
    const int vb = rest % W;
    const int chain = (rest / W) * 8 + xcd;
    if (chain >= p.n_chains) return;
    const int h = chain % H;
    int n = chain / H;
    if (p.cu_seqlens && p.n_chains / H <= kLptMaxSeqs)
        n = __builtin_amdgcn_readfirstlane(
            seq_of_rank(p.cu_seqlens, p.n_chains / H, n, threadIdx.x & 63));
    // the state slot of (sequence n, head h); the dispatch index `chain`
    // differs from it once sequences are dealt longest first
    const int64_t state_of = (int64_t)n * H + h;
    int64_t bos, T;
    if (p.cu_seqlens) {
        // entries are clamped into [0, n_tokens]: a cu_seqlens that breaks
        // its contract changes the result, never the addresses touched
        const int32_t c0 = p.cu_seqlens[n], c1 = p.cu_seqlens[n + 1];
        const int32_t a0 = c0 < 0 ? 0 : (c0 > p.n_tokens ? p.n_tokens : c0);
        const int32_t a1 = c1 < 0 ? 0 : (c1 > p.n_tokens ? p.n_tokens : c1);
        bos = a0;
        T = a1 > a0 ? a1 - a0 : 0;
    } else {
        bos = (int64_t)n * p.seqlen;
        T = p.seqlen;
    }
    // this job's tokens, its value source, entry state, output and final
    // state (all wave-uniform)
    const bool trans = vb >= NB;                 // transition columns of a later segment
    const int col_base = (trans ? vb - NB : vb) * C::BV;
    int64_t t0 = 0;                              // first token, relative to bos
    int s0_mode = p.S0 ? 1 : 0;                  // 0 zero, 1 load, 2 identity
    const float *s0p = p.S0 + state_of * DK * DV + col_base;
    int s0_row = DV;
    char *obase = reinterpret_cast<char *>(p.o);
    int64_t orow = (int64_t)H * DV * sizeof(TO), ocol = ((int64_t)h * DV + col_base) * sizeof(TO);
    bool out_f32 = sizeof(TO) == 4;
    float *stp = p.S_T ? p.S_T + state_of * DK * DV + col_base : nullptr;
    int st_row = DV;
    if (p.nseg > 1) {
        if (seg == 0) {
            T = T < p.len0 ? T : p.len0;
            stp = p.entry + state_of * (p.nseg - 1) * DK * DV + col_base;
        } else {
            t0 = p.len0 + (int64_t)(seg - 1) * p.lenS;
            const int64_t rem = T - t0;
            T = rem < 0 ? 0 : (rem < p.lenS ? rem : p.lenS);
            const int64_t aug = (int64_t)n * (p.seqlen - p.len0) + (t0 - p.len0);
            s0_mode = trans ? 2 : 0;
            st_row = DV + DK;
            stp = p.sumst + (state_of * (p.nseg - 1) + seg - 1) * DK * (DV + DK) +
                  (trans ? DV : 0) + col_base;
            out_f32 = true;
            if (trans) {
                obase = reinterpret_cast<char *>(p.rq + aug * H * DK);
                orow = (int64_t)H * DK * 4;
                ocol = ((int64_t)h * DK + col_base) * 4;
            } else {
                obase = reinterpret_cast<char *>(p.o0 + aug * H * DV);
                orow = (int64_t)H * DV * 4;
                ocol = ((int64_t)h * DV + col_base) * 4;
            }
        }
    }
    if (seg == 0) obase += bos * orow;
    bos += t0;
    // wave-uniform values are made visibly uniform (readfirstlane) so that
    // branches on them are scalar and the buffer resources built from them
    // live in scalar registers
    bos = uniform64(bos);
    const int Tn = __builtin_amdgcn_readfirstlane((int)T);     // < 2^31 - 64 (host)
    const int nch = (Tn + 15) / 16;
    // transition columns have zero values: their value loads get an empty
    // buffer range (they read zeros, as the ragged tail does)
    const bool v_on = !trans;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // roles: consumer waves 0 .. NW-1, builder waves NW .. NW+NBW-1, two helpers
    const bool is_cons = wave < NW;
    const bool is_build = !is_cons && wave < NW + C::NBW;
    const bool is_aux = C::AUX && wave >= NW + C::NBW + 2;
    const int bw = wave - NW, btid = tid - C::NC;     // builder wave / thread index
    const int j = lane & 15, g4 = lane >> 4;

    auto ntok_of = [&](int cc) -> int {
        const int rem = Tn - 16 * cc;
        return rem < 0 ? 0 : (rem < 16 ? rem : 16);
    };
    // Ring slot s.  The slot offset goes through readfirstlane, so every LDS
    // address is formed as (uniform slot base + per-lane offset + constant)
    // rather than carried as one pointer per access pattern across the loop.
    auto slot = [&](int s) -> Buf<C> & { return sm.buf[__builtin_amdgcn_readfirstlane(s)]; };

    // Pipeline over chunks with a ring of NBUF = 3 operand slots, in phases
    // separated by barriers (every role passes the same nch + 2 barriers):
    //   phase 0       builders build chunks 0 and 1
    //   phase 1       helpers form A, P, T of chunk 0
    //   phase 2 + c   builders build chunk c + 2 (slot (c + 2) % 3), helpers
    //                 form A, P, T of chunk c + 1 (slot (c + 1) % 3),
    //                 consumers store O of chunk c - 1 and run the S chain
    //                 of chunk c (slot c % 3)
    // Each SIMD holds one consumer and one builder wave, so the builder's
    // VALU work fills the consumer's matrix-core and LDS waits; the two
    // helper waves sit on SIMDs 0 and 1 and, where the configuration has
    // them, the two auxiliary waves on SIMDs 2 and 3 (the value block on the
    // builders' schedule, the Kd^T rows on the helpers').  Every role runs
    // its own loop over the same barriers; the role is wave-uniform.
    static_assert(NBUF == 3 && LAG == 2, "phase plan");
    if (is_build) {
        // Loads are issued unconditionally: buffer resources of chunks past
        // the end are empty and read zeros.  NR register sets take chunks in
        // turn (chunk cc in set cc % NR), so a chunk's loads are issued NR
        // phases before its build: at one chunk per phase, the loads have
        // NR phases to arrive, and NR sets of raw inputs are in flight.
        constexpr int NR = C::NR;
        Raw<C> r[NR];
        const void *gsrc = GATED ? static_cast<const void *>(p.z) : p.g;
        const void *bsrc = GATED ? static_cast<const void *>(p.braw) : p.beta;
        // e^A of this head (gated prologue)
        const float ea = GATED ? fast_exp2(p.A_log[h] * LOG2E) : 1.f;
        auto load = [&](Raw<C> &x, int cc) {
            load_raw<C>(x, p.q, p.k, p.v, gsrc, bsrc, bos + 16 * (int64_t)cc, ntok_of(cc),
                        v_on ? ntok_of(cc) : 0, H, h, DV, col_base, bw, lane, btid);
        };
#pragma unroll
        for (int i = 0; i < NR; ++i) load(r[i], i);
        if (nch > 0) build<C>(sm.buf[0], r[0], bw, lane, btid, ea);
        load(r[0], NR);
        if (nch > 1) build<C>(sm.buf[1], r[1], bw, lane, btid, ea);
        load(r[1], NR + 1);
        __syncthreads();
        __syncthreads();
        // phase 2 + cc builds chunk cc + 2 from set (cc + 2) % NR and refills
        // that set with chunk cc + 2 + NR.  The loop body is NR phases (c is
        // a multiple of NR, so every set index is a constant) and the last
        // nch % NR phases are peeled: every path back to the loop head has
        // issued the sets' loads in the same order, so the compiler's counter
        // waits keep the newer sets in flight.
        int c = 0;
#pragma unroll 1
        for (; c + NR <= nch; c += NR) {
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                if (c + i + 2 < nch) build<C>(slot((c + i + 2) % 3), r[(i + 2) % NR], bw, lane, btid, ea);
                load(r[(i + 2) % NR], c + i + 2 + NR);
                __syncthreads();
            }
        }
#pragma unroll
        for (int i = 0; i < NR - 1; ++i) {
            if (c + i < nch) {
                if (c + i + 2 < nch) build<C>(slot((c + i + 2) % 3), r[(i + 2) % NR], bw, lane, btid, ea);
                __syncthreads();
            }
        }
    } else if (is_aux) {
        if constexpr (C::AUX) {
            // the value block of chunk c + 2 (loads three phases ahead, like
            // the builders') and the Kd^T rows of chunk c + 1, whose Kd rows
            // the builders wrote a phase earlier
            const int a = tid - (NW + C::NBW + 2) * WAVE;
            constexpr int NR = 3;
            AuxV r[NR];
            AuxQK rn[GATED ? NR : 1];
            auto load = [&](int i, int cc) {
                aux_load_v<C>(r[i], p.v, bos + 16 * (int64_t)cc, v_on ? ntok_of(cc) : 0, H, h, DV,
                              col_base, a);
                if constexpr (GATED) aux_load_qk<C>(rn[i], p.q, p.k, bos + 16 * (int64_t)cc, ntok_of(cc), H, h, a);
            };
            auto write = [&](Buf<C> &B, int i) {
                aux_write_v<C>(B, r[i], a);
                if constexpr (GATED) aux_norms<C>(B, rn[i], a);
            };
#pragma unroll
            for (int i = 0; i < NR; ++i) load(i, i);
            if (nch > 0) write(sm.buf[0], 0);
            load(0, NR);
            if (nch > 1) write(sm.buf[1], 1);
            load(1, NR + 1);
            __syncthreads();
            if (nch > 0) aux_kh<C>(sm.buf[0], a);
            __syncthreads();
            int c = 0;
#pragma unroll 1
            for (; c + NR <= nch; c += NR) {
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    if (c + i + 2 < nch) write(slot((c + i + 2) % 3), (i + 2) % NR);
                    load((i + 2) % NR, c + i + 2 + NR);
                    if (c + i + 1 < nch) aux_kh<C>(slot((c + i + 1) % 3), a);
                    __syncthreads();
                }
            }
#pragma unroll
            for (int i = 0; i < NR - 1; ++i) {
                if (c + i < nch) {
                    if (c + i + 2 < nch) write(slot((c + i + 2) % 3), (i + 2) % NR);
                    if (c + i + 1 < nch) aux_kh<C>(slot((c + i + 1) % 3), a);
                    __syncthreads();
                }
            }
        }
    } else if (!is_cons) {
        // two helper waves on different SIMDs: A and T, and P
        auto help = [&](Buf<C> &B) {
            if (wave == NW + C::NBW) helper<C, 0>(B, lane);
            else helper<C, 1>(B, lane);
        };
        __syncthreads();
        if (nch > 0) help(sm.buf[0]);
        __syncthreads();
#pragma unroll 1
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) help(slot((c + 1) % 3));
            __syncthreads();
        }
    } else {
        // consumer state: S[:, col_base + 16 wave + j], rows 16 t + 4 g4 + i
        f32x4 S[DK / 16];
        const int col = 16 * wave + j;           // column inside the block
#pragma unroll
        for (int t = 0; t < DK / 16; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * t + 4 * g4 + i;
                S[t][i] = s0_mode == 1 ? s0p[(int64_t)row * s0_row + col]
                        : s0_mode == 2 ? (row == col_base + col ? 1.f : 0.f) : 0.f;
            }
        // O of chunk c is written at the start of iteration c + 1, so the
        // stores overlap the next chain instead of delaying this one.
        // lane (j, g4) holds O[token j][columns 16 wave + 4 g4 .. + 3]
        const int ow = (int)orow;                // < 2^31 / 16 (host)
        const int ooff = j * ow + (int)ocol + (16 * wave + 4 * g4) * (out_f32 ? 4 : (int)sizeof(TO));
        f32x4 ov = {0.f, 0.f, 0.f, 0.f};
        auto store_o = [&](int cc) {
            const rsrc_t ro = make_rsrc(obase + 16 * (int64_t)cc * orow,
                                        (cc >= 0 && !CKPT ? ntok_of(cc) : 0) * ow);
            if (out_f32) bstore4(ro, ooff, ov, float{});
            else bstore4(ro, ooff, ov, TO{});
        };
        __syncthreads();
        __syncthreads();
        Ahead<C> ah;
        read_ahead<C>(sm.buf[0], ah, wave, lane);
        // checkpoint tiles of this wave's 16 columns, chunk 0 of the sequence:
        // the entry state in fp32 tiles, or (bf16, d_k >= 32) the decayed
        // entry state Sd as the consumer's bf16 hi/lo operands
        constexpr bool CKS = CKPT && C::BF && DK >= 32;
        f32x4 *ck = nullptr;
        if constexpr (CKPT)
            ck = reinterpret_cast<f32x4 *>(p.ckpt + ((bos / 16 + n) * H + h) * (int64_t)(DK * DV)) +
                 ((col_base / 16 + wave) * (DK / 16)) * WAVE + lane;
#pragma unroll 1
        for (int c = 0; c < nch; ++c) {
            store_o(c - 1);
            if constexpr (CKPT && !CKS) {
#pragma unroll
                for (int t = 0; t < DK / 16; ++t)   // read once, by the backward: streamed
                    __builtin_nontemporal_store(S[t], &ck[(int64_t)c * H * (DK * DV / 4) + t * WAVE]);
            }
            if constexpr (CKS)
                ov = consume<C, true>(slot(c % 3), S, ah, wave, lane,
                                      reinterpret_cast<u32x4 *>(ck + (int64_t)c * H * (DK * DV / 4)));
            else
                ov = consume<C>(slot(c % 3), S, ah, wave, lane);
            read_ahead<C>(slot((c + 1) % 3), ah, wave, lane);
            __syncthreads();
        }
        if (nch > 0) store_o(nch - 1);
        if (stp) {
#pragma unroll
            for (int t = 0; t < DK / 16; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    stp[(int64_t)(16 * t + 4 * g4 + i) * st_row + col] = S[t][i];
        }
    }
}

// ---------------------------------------------------------------------------
// Segment scan (sequence split): the entry states of segments 2 .. nseg-1
// and the final state.  E_1 is segment 0's final state; then
// E_{s+1} = M_s E_s + S~_s, with M_s and S~_s the transition and value
// columns of segment s's final state.  fp32 throughout.  One workgroup per
// (chain, block of 16 state columns); the columns of S are independent.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void kda_seg_scan_kernel(const float *__restrict__ sumst,
                                                          float *__restrict__ entry,
                                                          float *__restrict__ S_T,
                                                          int32_t nseg)
{
    constexpr int NCB = DV / 16;
    constexpr int PER = (DK * 16 + 255) / 256;   // state elements per thread
    // M_s staged per step with coalesced row reads; E the running entry
    // state of this block of 16 columns
    __shared__ float M[DK][DK + 1];
    __shared__ float E[DK][17];
    const int chain = blockIdx.x / NCB, cb = blockIdx.x % NCB;
    const int tid = threadIdx.x;
    const int64_t ebase = (int64_t)chain * (nseg - 1) * DK * DV + cb * 16;
    for (int e = tid; e < DK * 16; e += 256) E[e / 16][e % 16] = entry[ebase + (e / 16) * DV + e % 16];
    for (int s = 1; s < nseg; ++s) {
        const float *A = sumst + ((int64_t)chain * (nseg - 1) + s - 1) * DK * (DV + DK);
        for (int e = tid; e < DK * DK; e += 256)
            M[e / DK][e % DK] = A[(int64_t)(e / DK) * (DV + DK) + DV + e % DK];
        float acc[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + 256 * i;
            acc[i] = e < DK * 16 ? A[(int64_t)(e / 16) * (DV + DK) + cb * 16 + e % 16] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + 256 * i;
            if (e < DK * 16) {
                const int r = e / 16, c = e % 16;
                float a = acc[i];
#pragma unroll 8
                for (int kk = 0; kk < DK; ++kk) a = __builtin_fmaf(M[r][kk], E[kk][c], a);
                acc[i] = a;
            }
        }
        __syncthreads();
        float *dst = s < nseg - 1 ? entry + ebase + (int64_t)s * DK * DV
                   : (S_T ? S_T + (int64_t)chain * DK * DV + cb * 16 : nullptr);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + 256 * i;
            if (e < DK * 16) {
                E[e / 16][e % 16] = acc[i];
                if (dst) dst[(e / 16) * DV + e % 16] = acc[i];
            }
        }
        // the next step's M and E reads follow its own barrier
    }
}

// ---------------------------------------------------------------------------
// Segment correction (sequence split): o_t = o~_t + E_s^T R_t for every
// token t of segment s >= 1, E_s its entry state, stored in the output type.
// Formed as O^T = E_s^T R^T on the bf16 matrix cores with hi/lo pairs of
// both operands (Eh Rh + El Rh + Eh Rl per 32-deep step; the dropped El Rl
// is near 2^-16 relative), so each lane ends with four consecutive outputs
// of one token.  One workgroup of eight waves per (chain, segment,
// kCorrTile tokens); E_s^T is staged in LDS as bf16 hi and lo rows.  A wave
// takes 16 tokens at a time and requests all of their R and o~ before its
// products (eight waves, so that enough loads are in flight per unit).
// ---------------------------------------------------------------------------
constexpr int kCorrTile = 256;                  // tokens per correction workgroup
static_assert(kCorrTile % 128 == 0, "eight waves of 16 tokens per step");
template <typename TO, int DK, int DV>
__global__ __launch_bounds__(512) void kda_seg_correct_kernel(
    TO *__restrict__ o, const float *__restrict__ o0, const float *__restrict__ rq,
    const float *__restrict__ entry, int32_t H, int32_t seqlen, int32_t len0, int32_t lenS,
    int32_t nseg, int32_t tiles)
{
    static_assert(DK % 32 == 0 && DV % 16 == 0, "correction tiles");
    // row stride 2 DK + 32 bytes, an odd multiple of 32: the 16-byte operand
    // reads below are free of bank conflicts
    constexpr int LE = DK + 16;
    __shared__ __attribute__((aligned(16))) bf16 EH[DV][LE];
    __shared__ __attribute__((aligned(16))) bf16 EL[DV][LE];
    const int tile = blockIdx.x % tiles;
    const int cs = blockIdx.x / tiles;
    const int seg = 1 + cs % (nseg - 1);
    const int chain = cs / (nseg - 1);            // n * H + h
    const int n = chain / H, h = chain % H;
    const int t0 = len0 + (seg - 1) * lenS;       // segment start inside the sequence
    int segT = seqlen - t0;
    segT = segT < lenS ? segT : lenS;
    const int tb = kCorrTile * tile;
    if (tb >= segT) return;
    const int ntile = segT - tb < kCorrTile ? segT - tb : kCorrTile;

    // E_s^T as hi/lo bf16: thread takes rows r, r + 1 of one column c
    const float *E = entry + ((int64_t)chain * (nseg - 1) + seg - 1) * DK * DV;
    for (int e = threadIdx.x; e < DK * DV / 2; e += 512) {
        const int c = e % DV, r = 2 * (e / DV);
        const float x0 = E[r * DV + c], x1 = E[(r + 1) * DV + c];
        const uint32_t hw = pack2(x0, x1);
        const bf16x2 hv = __builtin_bit_cast(bf16x2, hw);
        const uint32_t lw = pack2(x0 - (float)hv[0], x1 - (float)hv[1]);
        *reinterpret_cast<uint32_t *>(&EH[c][r]) = hw;
        *reinterpret_cast<uint32_t *>(&EL[c][r]) = lw;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nn = lane & 15, kg = lane >> 4;
    const int64_t aug0 = (int64_t)n * (seqlen - len0) + (t0 - len0) + tb;  // o~ / R row
    const int64_t tok0 = (int64_t)n * seqlen + t0 + tb;                     // o row
#pragma unroll 1
    for (int it = 0; it < kCorrTile / 128; ++it) {
        const int tt = 128 * it + 16 * wave;
        if (tt >= ntile) break;
        const int nt = ntile - tt < 16 ? ntile - tt : 16;
        const rsrc_t rr = make_rsrc(rq + (aug0 + tt) * H * DK, nt * H * DK * 4);
        const rsrc_t r0 = make_rsrc(o0 + (aug0 + tt) * H * DV, nt * H * DV * 4);
        const rsrc_t ro = make_rsrc(o + (tok0 + tt) * H * DV, nt * H * DV * (int)sizeof(TO));
        // every load of the 16 tokens first: R (lane (token nn, kg) holds
        // R[nn][32 s + 8 kg .. + 7], the B operand R^T) and o~ (lane (token
        // nn, kg) accumulates O[nn][16 ct + 4 kg .. + 3])
        f32x4 ra[DK / 32], rb[DK / 32], acc[DV / 16];
#pragma unroll
        for (int s2 = 0; s2 < DK / 32; ++s2) {
            const int off = ((nn * H + h) * DK + 32 * s2 + 8 * kg) * 4;
            ra[s2] = __builtin_bit_cast(f32x4, bload128(rr, off));
            rb[s2] = __builtin_bit_cast(f32x4, bload128(rr, off + 16));
        }
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct)
            acc[ct] = __builtin_bit_cast(f32x4, bload128(r0, ((nn * H + h) * DV + 16 * ct + 4 * kg) * 4));
        bf16x8 rh[DK / 32], rl[DK / 32];
#pragma unroll
        for (int s2 = 0; s2 < DK / 32; ++s2) {
            const f32x4 a = ra[s2], b = rb[s2];
            const u32x4 hw = {pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(b[0], b[1]),
                              pack2(b[2], b[3])};
            rh[s2] = __builtin_bit_cast(bf16x8, hw);
            f32x4 da, db;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                da[i] = a[i] - (float)rh[s2][i];
                db[i] = b[i] - (float)rh[s2][4 + i];
            }
            const u32x4 lw = {pack2(da[0], da[1]), pack2(da[2], da[3]), pack2(db[0], db[1]),
                              pack2(db[2], db[3])};
            rl[s2] = __builtin_bit_cast(bf16x8, lw);
        }
#pragma unroll
        for (int ct = 0; ct < DV / 16; ++ct) {
            const int ocol = (nn * H + h) * DV + 16 * ct + 4 * kg;
#pragma unroll
            for (int s2 = 0; s2 < DK / 32; ++s2) {
                const bf16x8 ah = ld8b(&EH[16 * ct + nn][32 * s2 + 8 * kg]);
                const bf16x8 al = ld8b(&EL[16 * ct + nn][32 * s2 + 8 * kg]);
                acc[ct] = mma32(ah, rh[s2], acc[ct]);
                acc[ct] = mma32(al, rh[s2], acc[ct]);
                acc[ct] = mma32(ah, rl[s2], acc[ct]);
            }
            bstore4(ro, ocol * (int)sizeof(TO), acc[ct], TO{});
        }
    }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
// waves per workgroup: 16 columns per consumer wave, at most 4 consumers and
// no more than the builder waves (each builder thread moves at most one
// four-token column piece of the value block)
template <int DK, int DV>
struct PickNW {
    static constexpr int byv = DV / 16 < 4 ? DV / 16 : 4;
    static constexpr int bydk = DK / 16;
    static constexpr int value = byv < bydk ? byv : bydk;
};

// Sequence-split plan.  Chunk counts; the segments are chunk-aligned.
struct SplitPlan {
    int nseg = 1, len0 = 0, lenS = 0;            // tokens
    size_t off_sumst = 0, off_entry = 0, off_o0 = 0, off_rq = 0, bytes = 0;
};

static int device_cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 256;
    return n > 0 ? n : 256;
}

// Finish time, in chunks, of the jobs one XCD runs: `cx` chains, each with
// `nb` jobs of segment 0 (l0 chunks) and, per later segment, `na` jobs of
// that segment's length; jobs start in order on the first free of `slots`
// compute units (one workgroup per unit: the LDS ring takes most of it).
static long long sim_makespan(int cx, int slots, int nb, int na, int nseg, long long L,
                              long long l0, long long ls)
{
    std::vector<long long> free_at((size_t)slots, 0);
    auto run = [&](long long len) {
        size_t best = 0;
        for (size_t i = 1; i < free_at.size(); ++i)
            if (free_at[i] < free_at[best]) best = i;
        free_at[best] += len;
    };
    for (int j = 0; j < cx * nb; ++j) run(l0 < L ? l0 : L);
    for (int s = 1; s < nseg; ++s) {
        long long len = L - l0 - (long long)(s - 1) * ls;
        len = len < 0 ? 0 : (len < ls ? len : ls);
        for (int j = 0; j < cx * na; ++j) run(len);
    }
    long long m = 0;
    for (long long f : free_at) m = f > m ? f : m;
    return m;
}

// Plans are cached per shape and device size: the search below runs a few
// hundred list-schedule simulations.
static std::mutex g_plan_mu;
static std::map<std::tuple<int, int, int, int, int, int>, SplitPlan> g_plans;

template <int DK, int DV>
static SplitPlan make_plan(const PrefillArgs &a)
{
    SplitPlan pl;
    if (a.cu_seqlens || DK < 32 || a.n_seqs <= 0 || a.seqlen < 1024) return pl;
    constexpr int NW = PickNW<DK, DV>::value;
    constexpr int BV = 16 * NW;
    constexpr int NB = DV / BV, NA = NB + DK / BV;
    const int cus = device_cus();
    const auto key = std::make_tuple(a.n_seqs, a.seqlen, a.H, DK, DV, cus);
    {
        std::lock_guard<std::mutex> lk(g_plan_mu);
        auto it = g_plans.find(key);
        if (it != g_plans.end()) return it->second;
    }
    const long long chains = (long long)a.n_seqs * a.H;
    const int slots = cus / 8 > 0 ? cus / 8 : 1;
    const int cx = (int)((chains + 7) / 8);       // chains on the busiest XCD
    const long long L = (a.seqlen + 15) / 16;
    // cost model, in microseconds, from MI355X kernel traces at d = 128: a
    // chunk step of a workgroup (about 1.4 us with every unit busy), the
    // correction streaming o~ and R in and o out at about 3.5 TB/s (the plan
    // does not depend on the output type), a scan step, two extra launches
    const double t_chunk = 1.4;
    auto cost = [&](long long mk, long long aug_tokens, int ns) {
        double c = (double)mk * t_chunk;
        if (aug_tokens > 0)
            c += (double)aug_tokens * a.H * (DV * 4 + DK * 4 + DV * 2) / 3.5e6 + 3.0 * ns + 10.0;
        return c;
    };
    double best = cx * NB <= slots ? cost(L, 0, 1)
                                   : cost(sim_makespan(cx, slots, NB, NA, 1, L, L, 0), 0, 1);
    const double base = best;
    if (cx * NB * 2 <= slots) {   // at most half of an XCD busy: a split can pay
        for (int nseg = 2; nseg <= 32; ++nseg) {
            for (int f = 1; f < 40; ++f) {
                const long long l0 = (L * f + 39) / 40;
                if (l0 >= L) continue;
                const long long ls = (L - l0 + nseg - 2) / (nseg - 1);
                if (ls < 8) continue;
                const int ns = 1 + (int)((L - l0 + ls - 1) / ls);   // no empty segment
                const long long mk = sim_makespan(cx, slots, NB, NA, ns, L, l0, ls);
                const long long aug = (long long)a.n_seqs * (a.seqlen - 16 * l0);
                const double c = cost(mk, aug, ns);
                if (c < best) {
                    best = c;
                    pl.nseg = ns;
                    pl.len0 = (int)(16 * l0);
                    pl.lenS = (int)(16 * ls);
                }
            }
        }
        if (best > 0.9 * base) pl = SplitPlan{};   // not worth the extra passes
    }
    if (pl.nseg > 1) {
        auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
        const size_t segs = (size_t)chains * (pl.nseg - 1);
        const size_t aug = (size_t)a.n_seqs * (a.seqlen - pl.len0) * a.H;
        pl.off_sumst = 0;
        pl.off_entry = up(segs * DK * (DV + DK) * 4);
        pl.off_o0 = pl.off_entry + up(segs * DK * DV * 4);
        pl.off_rq = pl.off_o0 + up(aug * DV * 4);
        pl.bytes = pl.off_rq + up(aug * DK * 4);
    }
    std::lock_guard<std::mutex> lk(g_plan_mu);
    g_plans[key] = pl;
    return pl;
}

template <typename TI, typename TO, int DK, int DV, int NW, int NBUF, bool GATED, bool CKPT>
static hipError_t launch_t(const PrefillArgs &a, int64_t chains, const SplitPlan &pl)
{
    using C = Cfg<TI, DK, NW, NBUF, GATED>;
    static_assert(DV % C::BV == 0, "column blocks");
    constexpr int NB = DV / C::BV, NA = NB + DK / C::BV;
    const int64_t chains8 = ((chains + 7) / 8) * 8;
    const int64_t grid = chains8 * (NB + (int64_t)(pl.nseg - 1) * NA);
    if (grid * C::NT >= ((int64_t)1 << 32)) return hipErrorInvalidValue;  // grid size limit
    if (pl.nseg > 1 && chains * (pl.nseg - 1) * ((pl.lenS + kCorrTile - 1) / kCorrTile) * 512 >= ((int64_t)1 << 32))
        return hipErrorInvalidValue;                                       // correction grid
    Params<TI, TO> p{};
    p.q = (const TI *)a.q; p.k = (const TI *)a.k; p.v = (const TI *)a.v;
    p.g = a.g; p.beta = a.beta; p.S0 = a.S0; p.cu_seqlens = a.cu_seqlens;
    p.o = (TO *)a.o; p.S_T = a.S_T;
    p.seqlen = a.seqlen; p.n_tokens = (int32_t)a.n_tokens;
    p.n_chains = (int32_t)chains; p.chains8 = (int32_t)chains8; p.H = a.H;
    p.nseg = pl.nseg; p.len0 = pl.len0; p.lenS = pl.lenS;
    p.z = (const TI *)a.z; p.braw = (const TI *)a.b; p.A_log = a.A_log;
    p.ckpt = a.ckpt;
    if (pl.nseg > 1) {
        char *ws = static_cast<char *>(a.workspace);
        p.sumst = reinterpret_cast<float *>(ws + pl.off_sumst);
        p.entry = reinterpret_cast<float *>(ws + pl.off_entry);
        p.o0 = reinterpret_cast<float *>(ws + pl.off_o0);
        p.rq = reinterpret_cast<float *>(ws + pl.off_rq);
    }
    hipStream_t st = (hipStream_t)a.stream;
    hipLaunchKernelGGL((kda_prefill_kernel<TI, TO, DK, DV, NW, NBUF, GATED, CKPT>), dim3((unsigned)grid),
                       dim3(C::NT), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.nseg == 1) return e;
    if (a.S_T || pl.nseg > 2) {
        hipLaunchKernelGGL((kda_seg_scan_kernel<DK, DV>), dim3((unsigned)(chains * (DV / 16))),
                           dim3(256), 0, st, p.sumst, p.entry, a.S_T, pl.nseg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if constexpr (DK % 32 == 0) {
        const int tiles = (pl.lenS + kCorrTile - 1) / kCorrTile;
        const int64_t g2 = chains * (pl.nseg - 1) * tiles;
        hipLaunchKernelGGL((kda_seg_correct_kernel<TO, DK, DV>), dim3((unsigned)g2), dim3(512), 0,
                           st, (TO *)a.o, p.o0, p.rq, p.entry, a.H, a.seqlen, pl.len0, pl.lenS,
                           pl.nseg, tiles);
        e = hipGetLastError();
    }
    return e;
}

template <typename TI, typename TO, int DK, int DV, bool GATED, bool CKPT>
static hipError_t launch_dims(const PrefillArgs &a)
{
    constexpr int NW = PickNW<DK, DV>::value;
    const int64_t chains = (int64_t)a.n_seqs * a.H;
    if (chains == 0) return hipSuccess;
    if (chains > INT32_MAX - 8) return hipErrorInvalidValue;
    static_assert(sizeof(Smem<Cfg<TI, DK, NW, 3, GATED>>) <= 160 * 1024, "LDS");
    SplitPlan pl;
    if (!CKPT && a.workspace) {
        pl = make_plan<DK, DV>(a);
        if (pl.bytes > a.workspace_bytes) pl = SplitPlan{};   // (checked by the caller)
    }
    return launch_t<TI, TO, DK, DV, NW, 3, GATED, CKPT>(a, chains, pl);
}

template <int DK, int DV>
static size_t plan_bytes(const PrefillArgs &a)
{
    return make_plan<DK, DV>(a).bytes;
}

#define KDA_PF_DIMS(X) \
    X(16, 16) X(16, 32) X(16, 64) X(16, 128) X(32, 16) X(32, 32) X(32, 64) X(32, 128) \
    X(64, 16) X(64, 32) X(64, 64) X(64, 128) X(128, 16) X(128, 32) X(128, 64) X(128, 128)

template <typename TI, typename TO, bool GATED, bool CKPT = false>
static hipError_t dispatch_dims(const PrefillArgs &a)
{
#define KDA_PF_CASE(DK_, DV_) \
    if (a.d_k == DK_ && a.d_v == DV_) return launch_dims<TI, TO, DK_, DV_, GATED, CKPT>(a);
    KDA_PF_DIMS(KDA_PF_CASE)
#undef KDA_PF_CASE
    return hipErrorInvalidValue;
}

size_t prefill_workspace_bytes(const PrefillArgs &a)
{
#define KDA_PF_CASE(DK_, DV_) \
    if (a.d_k == DK_ && a.d_v == DV_) return plan_bytes<DK_, DV_>(a);
    KDA_PF_DIMS(KDA_PF_CASE)
#undef KDA_PF_CASE
    return 0;
}

template <bool GATED>
static hipError_t dispatch_types(const PrefillArgs &a)
{
    if (a.in_bf16) {
        return a.out_bf16 ? dispatch_dims<bf16, bf16, GATED>(a)
                          : dispatch_dims<bf16, float, GATED>(a);
    }
    return dispatch_dims<float, float, GATED>(a);
}

hipError_t launch_prefill(const PrefillArgs &a)
{
    if (a.ckpt) {
        // checkpointing forward of the backward pass: g and beta given, no
        // output, no split
        if (a.gated) return hipErrorInvalidValue;
        return a.in_bf16 ? dispatch_dims<bf16, bf16, false, true>(a)
                         : dispatch_dims<float, float, false, true>(a);
    }
    return a.gated ? dispatch_types<true>(a) : dispatch_types<false>(a);
}

}  // namespace kda
