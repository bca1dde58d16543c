// Chunk-operand machinery shared by the KDA prefill and backward kernels
// (gfx950 / CDNA4 only): matrix-core wrappers and exact bf16 hi/lo splits,
// raw buffer resources for ragged tails, the per-chunk input loads, the
// builder that turns one chunk of q, k, g, beta (and a block of v or of dO)
// into end-referenced operands in LDS, and the helper waves that form the
// unit-lower inverse and the intra-chunk products on the matrix cores.
//
// The chunk algebra (every factor referenced to the chunk end) is stated at
// the prefill kernel.  With BWD set (bf16 only) the builder and helpers lay
// the operands out for the reverse-mode sweep instead: -KE^T and QE^T as
// [channel][token] rows in place of Kd^T, T^T in place of T, P^T in place
// of P, and the block of dO in place of the block of v.
#pragma once

#include <type_traits>

#include "kda_device.h"

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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// two floats as one packed bf16 word, round to nearest even
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// Exact bf16 residuals on the matrix core, lane by lane.  In the 16x16x32
// bf16 product, lane (n, g) = (lane % 16, lane / 16) holds D[4 g + i][n] of
// the accumulator and B[8 g + i][n] of the B operand, and the A operand row
// m has its K slots 8 (m / 4) + (m % 4) held by lane (m, m / 4).  With A the
// negative identity placed on those slots (NegEye below), D = C - B' where
// B' are the four values the same lane put in its own slots 0..3: any four
// floats x of a lane and their bf16 roundings h give x - h in one product.
// The product -h is exact and x - h is representable in fp32 when h is the
// round-to-nearest of x, so the sum is exact; this costs one MFMA in place of
// the shift, mask and two subtractions per pair on the vector ALU.  The same
// identity placed on the slots 4..7 (b below) takes the residual of the four
// values in the lane's upper slots, so two tiles whose roundings share one
// 8-slot operand [h0 | h1] need no zero padding and no copies.
struct NegEye {
    bf16x8 a, b;
};
__device__ __forceinline__ NegEye neg_eye(int lane)
{
    const int m = lane & 15, kg = lane >> 4;
    NegEye e;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        e.a[i] = (i < 4 && m == 4 * kg + i) ? (bf16)-1.0f : (bf16)0.0f;
        e.b[i] = (i >= 4 && m == 4 * kg + i - 4) ? (bf16)-1.0f : (bf16)0.0f;
    }
    return e;
}
__device__ __forceinline__ void split4(f32x4 x, const NegEye &ne, bf16x4 &h, bf16x4 &l)
{
    h = __builtin_bit_cast(bf16x4, u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])});
    const f32x4 r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ne.a, cat(h, bf16x4{}), x, 0, 0, 0);
    l = __builtin_bit_cast(bf16x4, u32x2{pack2(r[0], r[1]), pack2(r[2], r[3])});
}
// hi/lo split of two D-layout tiles into the 8-slot operands [h0 | h1] and
// [l0 | l1]
__device__ __forceinline__ void split8(f32x4 x0, f32x4 x1, const NegEye &ne, bf16x8 &h, bf16x8 &l)
{
    h = __builtin_bit_cast(bf16x8, u32x4{pack2(x0[0], x0[1]), pack2(x0[2], x0[3]),
                                         pack2(x1[0], x1[1]), pack2(x1[2], x1[3])});
    const f32x4 r0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ne.a, h, x0, 0, 0, 0);
    const f32x4 r1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ne.b, h, x1, 0, 0, 0);
    l = __builtin_bit_cast(bf16x8, u32x4{pack2(r0[0], r0[1]), pack2(r0[2], r0[3]),
                                         pack2(r1[0], r1[1]), pack2(r1[2], r1[3])});
}
__device__ __forceinline__ int64_t uniform64(int64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
// value of x in lane `lane` (wave-uniform result)
__device__ __forceinline__ float bcast(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Raw buffer resources: an access at a byte offset >= num_records reads 0
// and a store there is dropped, so per-chunk resources sized to the chunk's
// real tokens mask the ragged tail without branches (and every load and
// store of the main loop is issued unconditionally).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;        // raw buffer, 32-bit data format
// bytes >= 0; the host keeps 16 rows of any tensor below 2^31 bytes
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int bytes)
{
    // the size is wave-uniform; readfirstlane keeps the resource in scalar
    // registers whatever form the compiler gives the arithmetic before it
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), kRsrcFlags);
}
__device__ __forceinline__ uint32_t bload32(rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 bload64(rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ u32x4 bload128(rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void bstore(rsrc_t r, int off, bf16 x)
{
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, x), r, off, 0, 0);
}
__device__ __forceinline__ void bstore(rsrc_t r, int off, float x)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, off, 0, 0);
}
// four consecutive elements in the output type
__device__ __forceinline__ void bstore4(rsrc_t r, int off, f32x4 x, bf16)
{
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])}, r, off,
                                          0, 0);
}
__device__ __forceinline__ void bstore4(rsrc_t r, int off, f32x4 x, float)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// configuration
// ---------------------------------------------------------------------------
// operand layouts: the forward chunk, the reverse-mode sweep, or the
// per-chunk gradient kernel of the backward pass
enum { MODE_FWD = 0, MODE_SWEEP = 1, MODE_CHUNK = 2 };

template <typename TI, int DK_, int NW_, int NBUF_, bool GATED_ = false, int MODE_ = MODE_FWD>
struct Cfg {
    static constexpr bool BF = std::is_same<TI, bf16>::value;
    // backward layouts (bf16 only, not gated): T^T and P^T in place of T and
    // P; the sweep adds -KE^T | QE^T rows, the chunk kernel fp32 copies of
    // the exponents, of (I + A)^{-1} and of KE Kd^T
    static constexpr bool BWD = MODE_ != MODE_FWD;
    static constexpr bool SWEEP = MODE_ == MODE_SWEEP;
    static constexpr bool CHUNK = MODE_ == MODE_CHUNK;
    static_assert(!BWD || (BF && !GATED_), "the backward layouts are bf16, ungated");
    // gated prologue: raw q, k, the gate pre-activation z and beta's
    // pre-activation b come in (in the input type); the kernel forms
    // g = -5 sigmoid(e^A z), beta = sigmoid(b) and the L2 scales of q, k
    static constexpr bool GATED = GATED_;
    using OT = typename std::conditional<BF, bf16, float>::type;   // LDS operand type
    static constexpr int DK = DK_;
    static constexpr int NW = NW_;                 // consumer waves
    // builder waves: up to four, each with at least 16 key channels; the
    // count does not depend on the block width, so narrow blocks (d_v of 16
    // or 32) keep the build rate
    static constexpr int NBW = DK / 16 < 4 ? DK / 16 : 4;
    static constexpr int NBUF = NBUF_;             // LDS operand ring depth
    static constexpr int BV = 16 * NW;             // state columns per workgroup
    // two auxiliary waves take the value block (and, in the forward, the
    // Kd^T rows) off the builders (bf16, d_k = 128 with four consumers: with
    // them every SIMD holds one consumer, one builder and one helper or
    // auxiliary wave, three waves as before)
    static constexpr bool AUX = BF && MODE_ != MODE_CHUNK && DK_ == 128 && NW_ == 4;
    static constexpr int NT = (NW + NBW + 2 + (AUX ? 2 : 0)) * WAVE;   // + 2 helpers
    static constexpr int NC = NW * WAVE;           // consumer threads
    static constexpr int NVT = 4 * BV;             // builder threads that move v (4 tokens each)
    static_assert(NVT <= NBW * WAVE && NVT % WAVE == 0, "value block mapping");
    // builder thread tid moves v
    static __device__ __forceinline__ bool all_v(int tid) { return NVT == NBW * WAVE || tid < NVT; }
    // LDS strides.  gfx950 serves a 16-byte LDS access in four groups of 16
    // lanes (the quads of equal bit parity inside each half wave) over 64
    // four-byte banks.  A read where lane (j, g) = (lane % 16, lane / 16)
    // takes 16 bytes at row j, byte 16 g of its row is then free of bank
    // conflicts exactly when the row stride is an odd multiple of 32 bytes;
    // every operand row below that is read this way has such a stride.
    //
    // [16][DK] operand rows (bf16, d_k >= 32): inside every block of 32
    // channels the channels are stored in the order 0-3, 16-19, 4-7, 20-23,
    // 8-11, 24-27, 12-15, 28-31 (kpos below), so the eight K slots of one
    // consumer lane in a 32-deep product (channels 4 g + i and 16 + 4 g + i)
    // are one 16-byte read
    static constexpr int LDK = !BF ? DK + 4 : DK < 32 ? DK + 8 : ((DK / 8) % 4 == 2 ? DK : DK + 16);
    // Kd^T, T and P rows: bf16 rows hold each group of four tokens as
    // [4 hi | 4 lo] (Kd^T), [4 hi | 4 hi] (T hi, P hi) or [4 lo | 4 lo] (T lo,
    // P lo),
    // so one 16-byte read is an MFMA operand; 96-byte rows
    static constexpr int LDT = BF ? 48 : 20;       // row stride of Kd^T [DK][16]
    static constexpr int LDP = BF ? 48 : 20;       // row stride of T and P [16][16]
    // v block stored transposed, [column][token]: a consumer lane reads its
    // four tokens of one column with one 8-byte read (48-byte rows)
    static constexpr int LVT = BF ? 24 : 20;
    // sweep: -KE^T and QE^T rows [channel][token], each 16 tokens as four
    // groups [4 hi | 4 lo], -KE^T in bf16 0..31 and QE^T in 32..63; 160-byte
    // rows (an odd multiple of 32 bytes)
    static constexpr int LKQ = 80;
    // builder: wave w owns CW key channels; lane = (channel pair, token group)
    static constexpr int CW = DK / NBW;
    static constexpr int CPW = CW / 2;
    static constexpr int NG = WAVE / CPW;
    static constexpr int TPG = 16 / NG;
    static constexpr int LO = BF ? 1 : 0;          // hi/lo split present
    static constexpr int NR = BF ? 3 : 2;          // builder raw-input register sets
    static_assert(CW >= 16 && CW <= 128, "builder mapping needs 16 <= d_k/NBW <= 128");
    static_assert(NG * TPG == 16, "token groups");
    static_assert(NBUF >= 3, "one barrier per chunk needs three ring slots");
};

template <class C>
struct alignas(16) Buf {
    // every array starts on a 16-byte boundary: the 8- and 16-byte LDS
    // accesses below rely on it, whichever arrays are placeholders (size 1)
    // in a given layout
    using OT = typename C::OT;
    alignas(16) OT NK[16][C::LDK];                   // -KE                  [token][channel]
    alignas(16) OT QH[16][C::LDK];                   // QE hi
    alignas(16) OT QL[C::LO ? 16 : 1][C::LDK];       // QE lo
    alignas(16) OT DH[16][C::LDK];                   // Kd hi                [token][channel]
    alignas(16) OT DL[C::LO ? 16 : 1][C::LDK];       // Kd lo
    alignas(16) OT KH[C::BWD ? 1 : C::DK][C::LDT];   // Kd^T                 [channel][token]
    alignas(16) OT KQ[C::SWEEP ? C::DK : 1][C::SWEEP ? C::LKQ : 1];   // sweep: -KE^T | QE^T
    alignas(16) OT TH[16][C::LDP];                   // T (hi); sweep: T^T   [token r][token i]
    alignas(16) OT TL[C::LO ? 16 : 1][C::LDP];       // T lo
    alignas(16) OT PH[16][C::LDP];                   // P (hi); sweep: P^T as [4 hi | 4 lo]
    alignas(16) OT PL[C::LO && !C::BWD ? 16 : 1][C::LDP];   // P lo
    alignas(16) OT VT[C::CHUNK ? 1 : C::BV][C::LVT]; // value block, transposed  [column][token]
    alignas(16) float DEC[C::DK];                    // e^{Gc_16} per channel
    alignas(16) float BETA[16];
    // gated prologue: per builder wave, the partial sums of q^2 and k^2 of
    // each token over its channels; then the scales 1 / |q|, 1 / |k|
    alignas(16) float NRM[C::GATED ? 2 : 1][C::GATED ? C::NBW : 1][16];
    alignas(16) float SQ[C::GATED ? 16 : 1], SK[C::GATED ? 16 : 1];
    // chunk kernel: Gc_r - Gc_16 (log2 units) [token][channel] (natural
    // channel order), (I + A)^{-1} and KE Kd^T
    static constexpr int NX = C::CHUNK ? 16 : 1, DX = C::CHUNK ? C::DK + 4 : 1;
    alignas(16) float GX[NX][DX];
    alignas(16) float MI[NX][17], KK[NX][17];
};

// stored position of key channel c in a [16][DK] operand row (see LDK)
template <class C>
__device__ __forceinline__ int kpos(int c)
{
    if constexpr (C::BF && C::DK >= 32) {
        const int q = (c >> 2) & 7;
        return (c & ~31) | ((q & 3) << 3) | ((q >> 2) << 2) | (c & 3);
    } else {
        return c;
    }
}

template <class C>
struct alignas(16) Smem {
    Buf<C> buf[C::NBUF];
};

// raw (un-scaled) chunk inputs held in registers between load and build,
// as the bits the buffer loads return (zero past the sequence end)
template <class C>
struct Raw {
    typedef typename std::conditional<C::BF, uint32_t, u32x2>::type P2;   // 2 q/k elements
    P2 q[C::TPG], k[C::TPG];
    // log-decay g (fp32 pairs) or, gated, the gate pre-activation z (as q)
    typename std::conditional<C::GATED, P2, u32x2>::type g[C::TPG];
    // 4 tokens of one v column (bf16: packed pairs, fp32: one per word)
    typename std::conditional<C::BF, u32x2, u32x4>::type v;
    uint32_t beta;
    int ntok;                             // real tokens of the chunk
};

template <class C>
__device__ __forceinline__ float elem(typename Raw<C>::P2 x, int i)
{
    if constexpr (C::BF) return u16_to_f(i ? (uint16_t)(x >> 16) : (uint16_t)(x & 0xffffu));
    else return __uint_as_float(x[i]);
}
// ---------------------------------------------------------------------------
// loads of one chunk's raw inputs through buffer resources bounded by the
// chunk's real tokens: padded tokens read k = q = v = 0, g = 0, beta = 0,
// an exact identity transition.  ntok may be <= 0 (nothing is read); the
// values are read for ntok_v tokens (ntok, or 0 for zero values).
// ---------------------------------------------------------------------------
template <class C, typename TI>
__device__ __forceinline__ void load_raw(Raw<C> &r, const TI *__restrict__ q,
                                         const TI *__restrict__ k, const TI *__restrict__ v,
                                         const void *__restrict__ g,
                                         const void *__restrict__ beta, int64_t tok_base,
                                         int ntok, int ntok_v, int H, int h, int DV,
                                         int col_base, int wave, int lane, int tid)
{
    constexpr int ES = sizeof(TI);
    // g and beta: fp32, or (gated) z and b in the input type
    constexpr int GS = C::GATED ? ES : 4;
    const int rowk = H * C::DK, rowv = H * DV;
    const rsrc_t rq = make_rsrc(q + tok_base * rowk, ntok * rowk * ES);
    const rsrc_t rk = make_rsrc(k + tok_base * rowk, ntok * rowk * ES);
    const rsrc_t rg = make_rsrc(static_cast<const char *>(g) + tok_base * rowk * GS,
                                ntok * rowk * GS);
    const rsrc_t rv = make_rsrc(v + tok_base * rowv, ntok_v * rowv * ES);
    const rsrc_t rb = make_rsrc(static_cast<const char *>(beta) + tok_base * H * GS,
                                ntok * H * GS);
    const int cp = lane % C::CPW, tg = lane / C::CPW;
    const int ch = wave * C::CW + 2 * cp;
    r.ntok = ntok;
#pragma unroll
    for (int t = 0; t < C::TPG; ++t) {
        const int e = (tg * C::TPG + t) * rowk + h * C::DK + ch;
        if constexpr (C::BF) {
            r.q[t] = bload32(rq, e * ES);
            r.k[t] = bload32(rk, e * ES);
        } else {
            r.q[t] = bload64(rq, e * ES);
            r.k[t] = bload64(rk, e * ES);
        }
        if constexpr (!C::GATED) r.g[t] = bload64(rg, e * 4);
        else if constexpr (C::BF) r.g[t] = bload32(rg, e * ES);
        else r.g[t] = bload64(rg, e * ES);
    }
    if constexpr (C::GATED && C::BF)
        r.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, ((tid & 15) * H + h) * ES, 0, 0);
    else
        r.beta = bload32(rb, ((tid & 15) * H + h) * 4);
    // v: thread (column c, token quad tq) < NVT loads tokens 4 tq .. 4 tq + 3
    // of column c (a wave's loads of one token are consecutive columns); the
    // condition is uniform over each wave and absent when all builders move v
    if constexpr (C::AUX) return;                  // the auxiliary waves move v
    if constexpr (C::CHUNK) return;                // the chunk kernel reads v itself
    if (!C::all_v(tid)) return;
    const int c = tid % C::BV, tq = tid / C::BV;
    const int ev = 4 * tq * rowv + h * DV + col_base + c;
    if constexpr (C::BF) {
        // 16-bit loads straight into the halves of two packed registers
        typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
        u16x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __builtin_amdgcn_raw_buffer_load_b16(rv, (ev + i * rowv) * ES, 0, 0);
        r.v = __builtin_bit_cast(u32x2, x);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[i] = bload32(rv, (ev + i * rowv) * ES);
    }
}

// ---------------------------------------------------------------------------
// Inclusive prefix sum over the NG token groups of a wave (group tg = lane /
// CPW, one value per lane and group) and the total over all groups.  The
// builder mapping gives NG = 4 (d_k = 128: the groups are the 16-lane rows,
// exchanged with the register swaps across row pairs and half waves, no LDS
// round trip) or NG = 8 (d_k <= 64: eight-lane groups, lane shuffles).
// ---------------------------------------------------------------------------
template <int NG, int CPW>
__device__ __forceinline__ void group_scan(float x, int tg, float &incl, float &tot)
{
    static_assert(NG == 4 || NG == 8, "builder token groups");
    if constexpr (NG == 4) {
        float ev, od;                    // the even and odd row of this row pair
        row_pair(x, ev, od);
        const float pair = ev + od;
        const float ip = (tg & 1) ? pair : x;
        float lo, hi;                    // pair totals of rows 0-1 and rows 2-3
        half_pair(pair, lo, hi);
        incl = (tg & 2) ? ip + lo : ip;
        tot = lo + hi;
    } else {
        incl = x;
#pragma unroll
        for (int off = 1; off < NG; off <<= 1) {
            const float n = __shfl_up(incl, off * CPW, WAVE);
            if (tg >= off) incl += n;
        }
        tot = __shfl(incl, (WAVE - CPW) + (__lane_id() % CPW), WAVE);
    }
}

// ---------------------------------------------------------------------------
// Sum over each aligned group of N = 8 or 16 lanes, left in every lane of the
// group: a butterfly of data-parallel-primitive lane moves inside a 16-lane
// row (swap neighbours, swap pairs, mirror the half row, mirror the row),
// each folded into a vector add; no LDS round trip.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    static_assert(N == 8 || N == 16, "lane groups of 8 or 16");
    x += dpp_mov<0xB1>(x);                        // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);                        // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);                       // row_half_mirror
    if constexpr (N == 16) x += dpp_mov<0x140>(x); // row_mirror
    return x;
}

// ---------------------------------------------------------------------------
// build: raw registers -> end-referenced operands of one chunk in LDS
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void build(Buf<C> &B, const Raw<C> &r, int wave, int lane, int tid,
                                      float ea)
{
    using OT = typename C::OT;
    typedef OT OT2 __attribute__((ext_vector_type(2)));
    constexpr int TPG = C::TPG;
    const int cp = lane % C::CPW, tg = lane / C::CPW;
    const int ch = wave * C::CW + 2 * cp;
    const int tok0 = tg * TPG;
    const int kc = kpos<C>(ch);           // stored position of the pair (ch, ch + 1)
    const NegEye ne = neg_eye(lane);

    // cumulative log2-decay over this lane's tokens, then across token groups
    float G0[TPG], G1[TPG];
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int t = 0; t < TPG; ++t) {
        if constexpr (C::GATED) {
            // g log2(e) = -5 log2(e) sigmoid(y), y = e^A z: the lower-bounded
            // gate (K3-on-TPU essay, "KDA + Gated MLA", lower-bounded decay);
            // y -> -inf gives exp2 = inf, rcp = 0, g = 0, the right limit
            // a padded token of the ragged tail must stay the identity (g = 0)
            const float y0 = ea * elem<C>(r.g[t], 0), y1 = ea * elem<C>(r.g[t], 1);
            const float live = tok0 + t < r.ntok ? -5.f * LOG2E : 0.f;
            s0 += live * __builtin_amdgcn_rcpf(1.f + fast_exp2(-y0 * LOG2E));
            s1 += live * __builtin_amdgcn_rcpf(1.f + fast_exp2(-y1 * LOG2E));
        } else {
            s0 = __builtin_fmaf(__uint_as_float(r.g[t][0]), LOG2E, s0);
            s1 = __builtin_fmaf(__uint_as_float(r.g[t][1]), LOG2E, s1);
        }
        G0[t] = s0;
        G1[t] = s1;
    }
    if constexpr (C::GATED && !C::AUX) {
        // partial |q|^2 and |k|^2 of this lane's tokens over the wave's
        // channels: sum the channel pairs of the CPW lanes of a token group
        // (with auxiliary waves, they form the whole sums instead)
#pragma unroll
        for (int t = 0; t < TPG; ++t) {
            const float qa = elem<C>(r.q[t], 0), qb = elem<C>(r.q[t], 1);
            const float ka = elem<C>(r.k[t], 0), kb = elem<C>(r.k[t], 1);
            float nq = qa * qa + qb * qb, nk = ka * ka + kb * kb;
            nq = group_sum<C::CPW>(nq);
            nk = group_sum<C::CPW>(nk);
            if (cp == 0) {
                B.NRM[0][wave][tok0 + t] = nq;
                B.NRM[1][wave][tok0 + t] = nk;
            }
        }
    }
    // inclusive scan of the group totals, and the chunk total Gc_16
    float i0, i1, T0, T1;
    group_scan<C::NG, C::CPW>(s0, tg, i0, T0);
    group_scan<C::NG, C::CPW>(s1, tg, i1, T1);
    // Gc_r - Gc_16 = (local prefix + exclusive offset) - total
    const float o0 = i0 - s0 - T0, o1 = i1 - s1 - T1;

    OT kdh0[TPG], kdh1[TPG], kdl0[TPG], kdl1[TPG];
    f32x4 qk[TPG];                        // QE and Kd of the channel pair, per token
    f32x2 nke[C::SWEEP ? TPG : 1];        // sweep: -KE of the channel pair, per token
    uint32_t qhw[C::SWEEP ? TPG : 1], qlw[C::SWEEP ? TPG : 1];   // sweep: QE hi, lo words
#pragma unroll
    for (int t = 0; t < TPG; ++t) {
        const int tok = tok0 + t;
        const float d0 = G0[t] + o0, d1 = G1[t] + o1;                 // >= 0 (log2)
        const float e0 = fast_exp2(d0), e1 = fast_exp2(d1);           // E
        const float f0 = fast_exp2(-d0), f1 = fast_exp2(-d1);         // 1 / E
        const float ka = elem<C>(r.k[t], 0), kb = elem<C>(r.k[t], 1);
        const float qa = elem<C>(r.q[t], 0), qb = elem<C>(r.q[t], 1);
        qk[t] = f32x4{qa * e0, qb * e1, ka * f0, kb * f1};
        if constexpr (C::SWEEP) nke[t] = f32x2{-ka * e0, -kb * e1};
        if constexpr (C::CHUNK) {
            *reinterpret_cast<f32x2 *>(&B.GX[tok][ch]) = f32x2{d0, d1};
        }
        if constexpr (C::BF) {
            *reinterpret_cast<uint32_t *>(&B.NK[tok][kc]) = pack2(-ka * e0, -kb * e1);
        } else {
            *reinterpret_cast<OT2 *>(&B.NK[tok][kc]) = OT2{-ka * e0, -kb * e1};
            *reinterpret_cast<OT2 *>(&B.QH[tok][kc]) = OT2{qk[t][0], qk[t][1]};
            *reinterpret_cast<OT2 *>(&B.DH[tok][kc]) = OT2{qk[t][2], qk[t][3]};
            kdh0[t] = qk[t][2]; kdh1[t] = qk[t][3];
        }
    }
    if constexpr (C::BF) {
        // QE and Kd of the channel pair as hi/lo bf16 pairs, two tokens per
        // split (words: QE hi, Kd hi of token t, then of token t + 1)
        static_assert(TPG % 2 == 0, "token pairs");
#pragma unroll
        for (int t = 0; t < TPG; t += 2) {
            bf16x8 h8, l8;
            split8(qk[t], qk[t + 1], ne, h8, l8);
            const u32x4 hw = __builtin_bit_cast(u32x4, h8), lw = __builtin_bit_cast(u32x4, l8);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tok = tok0 + t + u;
                const uint32_t qh = hw[2 * u], dh = hw[2 * u + 1];
                const uint32_t ql = lw[2 * u], dl = lw[2 * u + 1];
                *reinterpret_cast<uint32_t *>(&B.QH[tok][kc]) = qh;
                *reinterpret_cast<uint32_t *>(&B.QL[tok][kc]) = ql;
                *reinterpret_cast<uint32_t *>(&B.DH[tok][kc]) = dh;
                *reinterpret_cast<uint32_t *>(&B.DL[tok][kc]) = dl;
                if constexpr (C::SWEEP) {
                    qhw[t + u] = qh;
                    qlw[t + u] = ql;
                }
                const bf16x2 vh = __builtin_bit_cast(bf16x2, dh), vl = __builtin_bit_cast(bf16x2, dl);
                kdh0[t + u] = vh[0]; kdh1[t + u] = vh[1]; kdl0[t + u] = vl[0]; kdl1[t + u] = vl[1];
            }
        }
    }
    if constexpr (C::SWEEP) {
        // sweep: -KE^T and QE^T rows of channels ch, ch + 1 as hi/lo pairs;
        // -KE of a token pair is split in one go, QE's halves are the words
        // just stored to QH and QL
        bf16 nh0[TPG], nh1[TPG], nl0[TPG], nl1[TPG], qh0[TPG], qh1[TPG], ql0[TPG], ql1[TPG];
#pragma unroll
        for (int t = 0; t < TPG; t += 2) {
            bf16x4 h4, l4;
            split4(f32x4{nke[t][0], nke[t][1], nke[t + 1][0], nke[t + 1][1]}, ne, h4, l4);
            nh0[t] = h4[0]; nh1[t] = h4[1]; nh0[t + 1] = h4[2]; nh1[t + 1] = h4[3];
            nl0[t] = l4[0]; nl1[t] = l4[1]; nl0[t + 1] = l4[2]; nl1[t + 1] = l4[3];
        }
#pragma unroll
        for (int t = 0; t < TPG; ++t) {
            const bf16x2 hq = __builtin_bit_cast(bf16x2, qhw[t]);
            const bf16x2 lq = __builtin_bit_cast(bf16x2, qlw[t]);
            qh0[t] = hq[0]; qh1[t] = hq[1]; ql0[t] = lq[0]; ql1[t] = lq[1];
        }
        if constexpr (TPG == 2) {
            const int o = 8 * (tok0 >> 2) + (tok0 & 3);
            *reinterpret_cast<bf16x2 *>(&B.KQ[ch][o]) = bf16x2{nh0[0], nh0[1]};
            *reinterpret_cast<bf16x2 *>(&B.KQ[ch][o + 4]) = bf16x2{nl0[0], nl0[1]};
            *reinterpret_cast<bf16x2 *>(&B.KQ[ch + 1][o]) = bf16x2{nh1[0], nh1[1]};
            *reinterpret_cast<bf16x2 *>(&B.KQ[ch + 1][o + 4]) = bf16x2{nl1[0], nl1[1]};
            *reinterpret_cast<bf16x2 *>(&B.KQ[ch][32 + o]) = bf16x2{qh0[0], qh0[1]};
            *reinterpret_cast<bf16x2 *>(&B.KQ[ch][32 + o + 4]) = bf16x2{ql0[0], ql0[1]};
            *reinterpret_cast<bf16x2 *>(&B.KQ[ch + 1][32 + o]) = bf16x2{qh1[0], qh1[1]};
            *reinterpret_cast<bf16x2 *>(&B.KQ[ch + 1][32 + o + 4]) = bf16x2{ql1[0], ql1[1]};
        } else {
#pragma unroll
            for (int t = 0; t < TPG; t += 4) {
                const int o = 2 * (tok0 + t);
                *reinterpret_cast<bf16x8 *>(&B.KQ[ch][o]) =
                    bf16x8{nh0[t], nh0[t + 1], nh0[t + 2], nh0[t + 3],
                           nl0[t], nl0[t + 1], nl0[t + 2], nl0[t + 3]};
                *reinterpret_cast<bf16x8 *>(&B.KQ[ch + 1][o]) =
                    bf16x8{nh1[t], nh1[t + 1], nh1[t + 2], nh1[t + 3],
                           nl1[t], nl1[t + 1], nl1[t + 2], nl1[t + 3]};
                *reinterpret_cast<bf16x8 *>(&B.KQ[ch][32 + o]) =
                    bf16x8{qh0[t], qh0[t + 1], qh0[t + 2], qh0[t + 3],
                           ql0[t], ql0[t + 1], ql0[t + 2], ql0[t + 3]};
                *reinterpret_cast<bf16x8 *>(&B.KQ[ch + 1][32 + o]) =
                    bf16x8{qh1[t], qh1[t + 1], qh1[t + 2], qh1[t + 3],
                           ql1[t], ql1[t + 1], ql1[t + 2], ql1[t + 3]};
            }
        }
    } else if constexpr (C::CHUNK) {
        // the chunk kernel reads Kd from the fp32 copy
    } else if constexpr (C::AUX) {
        // the auxiliary waves write Kd^T from the Kd rows
    } else if constexpr (C::BF) {
        // Kd^T rows: this lane's TPG consecutive tokens of channels ch, ch + 1
        if constexpr (TPG == 2) {
            const int o = 8 * (tok0 >> 2) + (tok0 & 3);
            *reinterpret_cast<bf16x2 *>(&B.KH[ch][o]) = bf16x2{kdh0[0], kdh0[1]};
            *reinterpret_cast<bf16x2 *>(&B.KH[ch][o + 4]) = bf16x2{kdl0[0], kdl0[1]};
            *reinterpret_cast<bf16x2 *>(&B.KH[ch + 1][o]) = bf16x2{kdh1[0], kdh1[1]};
            *reinterpret_cast<bf16x2 *>(&B.KH[ch + 1][o + 4]) = bf16x2{kdl1[0], kdl1[1]};
        } else {
#pragma unroll
            for (int t = 0; t < TPG; t += 4) {
                const int o = 2 * (tok0 + t);
                *reinterpret_cast<bf16x8 *>(&B.KH[ch][o]) =
                    bf16x8{kdh0[t], kdh0[t + 1], kdh0[t + 2], kdh0[t + 3],
                           kdl0[t], kdl0[t + 1], kdl0[t + 2], kdl0[t + 3]};
                *reinterpret_cast<bf16x8 *>(&B.KH[ch + 1][o]) =
                    bf16x8{kdh1[t], kdh1[t + 1], kdh1[t + 2], kdh1[t + 3],
                           kdl1[t], kdl1[t + 1], kdl1[t + 2], kdl1[t + 3]};
            }
        }
    } else if constexpr (TPG == 2) {
        *reinterpret_cast<OT2 *>(&B.KH[ch][tok0]) = OT2{kdh0[0], kdh0[1]};
        *reinterpret_cast<OT2 *>(&B.KH[ch + 1][tok0]) = OT2{kdh1[0], kdh1[1]};
    } else {
        typedef OT OT4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int t = 0; t < TPG; t += 4) {
            *reinterpret_cast<OT4 *>(&B.KH[ch][tok0 + t]) =
                OT4{kdh0[t], kdh0[t + 1], kdh0[t + 2], kdh0[t + 3]};
            *reinterpret_cast<OT4 *>(&B.KH[ch + 1][tok0 + t]) =
                OT4{kdh1[t], kdh1[t + 1], kdh1[t + 2], kdh1[t + 3]};
        }
    }
    if (tg == 0) {
        B.DEC[ch] = fast_exp2(T0);
        B.DEC[ch + 1] = fast_exp2(T1);
    }
    {
        // v is stored in its input type (the raw bits): four tokens of one
        // column per thread, one 8- or 16-byte write
        const int c = tid % C::BV, tq = tid / C::BV;
        if (!C::AUX && !C::CHUNK && C::all_v(tid)) {
            if constexpr (C::BF) *reinterpret_cast<u32x2 *>(&B.VT[c][4 * tq]) = r.v;
            else *reinterpret_cast<u32x4 *>(&B.VT[c][4 * tq]) = r.v;
        }
    }
    if (tid < 16) {
        if constexpr (C::GATED) {
            // beta = sigmoid(b)
            const float b = C::BF ? u16_to_f((uint16_t)r.beta) : __uint_as_float(r.beta);
            B.BETA[tid] = __builtin_amdgcn_rcpf(1.f + fast_exp2(-b * LOG2E));
        } else {
            B.BETA[tid] = __uint_as_float(r.beta);
        }
    }
}

// ---------------------------------------------------------------------------
// 16x16 products on the matrix cores between tiles held in the accumulator
// (D) layout: lane (n, g) = (lane % 16, lane / 16) holds X[4 g + i][n].
// A tile in D layout is directly a B operand when its K index 4 g + i sits in
// the slots of group g; the left factor Y must then be given as Y^T in D
// layout (lane (r, g) holds Y[r][4 g + i]).  So prod(YT, X) = Y X and
// prod(X, YT) = X^T Y^T take the same two tiles with the roles swapped.
// bf16: one product, the K slots 4..7 of each group hold zeros.  fp32: four
// K=4 steps.
// ---------------------------------------------------------------------------
template <bool BF> struct Tile;
template <> struct Tile<true> {
    bf16x8 v;                            // [X (4 slots) | 0]
};
template <> struct Tile<false> {
    f32x4 x;
};
template <bool BF>
__device__ __forceinline__ Tile<BF> to_tile(f32x4 x)
{
    if constexpr (BF) {
        const u32x2 h = {pack2(x[0], x[1]), pack2(x[2], x[3])};
        return Tile<true>{cat(__builtin_bit_cast(bf16x4, h), bf16x4{})};
    } else {
        return Tile<false>{x};
    }
}
template <bool BF>
__device__ __forceinline__ f32x4 prod(const Tile<BF> &yt, const Tile<BF> &x)
{
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BF) {
        return mma32(yt.v, x.v, zero);
    } else {
        f32x4 r = zero;
#pragma unroll
        for (int s = 0; s < 4; ++s) r = mma4(yt.x[s], x.x[s], r);
        return r;
    }
}

// ---------------------------------------------------------------------------
// helper waves: A and T = (I + A)^{-1} Diag(beta) (PART 0), P (PART 1)
//
// A is strictly lower triangular, so A^16 = 0 and
//   (I + A)^{-1} = (I - A)(I + A^2)(I + A^4)(I + A^8)
// exactly (each factor pair telescopes: (I + A)(I - A) = I - A^2, ...).  The
// factors are polynomials in A and commute; the inverse is formed with
// eight 16x16 matrix-core products, keeping every intermediate in registers.
// With bf16 inputs A is itself formed from single-bf16 operands, and the
// products of the inverse take single-bf16 operands too (checked in
// emulation against the oracle: no change in the error of o or S_T); T is
// then written as a hi/lo pair.
// ---------------------------------------------------------------------------
template <class C, int PART>
__device__ __forceinline__ void helper(Buf<C> &B, int lane)
{
    using OT = typename C::OT;
    typedef OT OT4 __attribute__((ext_vector_type(4)));
    constexpr bool BF = C::BF;
    const int j = lane & 15, g4 = lane >> 4;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const NegEye ne = neg_eye(lane);
    // With M = KE Kd^T (M[t][s] = KE_t . Kd_s):
    //   mt[e] (lane (j, g4)) = -M[j][4 g4 + e]       (D layout of -M^T)
    //   mc[e] (lane (j, g4)) = -M[4 g4 + e][j]       (D layout of -M)
    //   pt[e] (lane (j, g4)) =  QE_j . Kd_{4 g4 + e} = P[j][4 g4 + e]
    f32x4 mt = zero, mc = zero, pt = zero;
    if constexpr (BF) {
        if constexpr (C::DK >= 32) {
            // K slot (g4, i) = stored position 32 s + 8 g4 + i, the same
            // channel on both operands
#pragma unroll
            for (int s = 0; s < C::DK / 32; ++s) {
                const int kk = 32 * s + 8 * g4;
                const bf16x8 dh = ld8b(&B.DH[j][kk]);
                if constexpr (PART == 0) {
                    const bf16x8 nk = ld8b(&B.NK[j][kk]);
                    mt = mma32(dh, nk, mt);
                    mc = mma32(nk, dh, mc);
                } else {
                    const bf16x8 qh = ld8b(&B.QH[j][kk]), ql = ld8b(&B.QL[j][kk]);
                    const bf16x8 dl = ld8b(&B.DL[j][kk]);
                    if constexpr (C::BWD) {
                        // operands swapped: the transposed product P^T
                        pt = mma32(qh, dh, pt);
                        pt = mma32(qh, dl, pt);
                        pt = mma32(ql, dh, pt);
                    } else {
                        pt = mma32(dh, qh, pt);
                        pt = mma32(dl, qh, pt);
                        pt = mma32(dh, ql, pt);
                    }
                }
            }
        } else {
            // d_k = 16: K slot (g4, i) = channel 4 g4 + i%4 of the hi (i < 4)
            // or lo (i >= 4) part
            const int kk = 4 * g4;
            const bf16x4 nk = ld4b(&B.NK[j][kk]);
            const bf16x4 qh = ld4b(&B.QH[j][kk]), ql = ld4b(&B.QL[j][kk]);
            const bf16x4 dh = ld4b(&B.DH[j][kk]);
            const bf16x8 dd = cat(dh, ld4b(&B.DL[j][kk]));
            const bf16x4 z = {};
            if constexpr (PART == 0) {
                mt = mma32(cat(dh, z), cat(nk, z), mt);
                mc = mma32(cat(nk, z), cat(dh, z), mc);
            } else if constexpr (C::BWD) {
                pt = mma32(cat(qh, qh), dd, pt);    // transposed: P^T
                pt = mma32(cat(ql, ql), dd, pt);
            } else {
                pt = mma32(dd, cat(qh, qh), pt);    // (dh + dl) qh
                pt = mma32(dd, cat(ql, ql), pt);    // (dh + dl) ql
            }
        }
    } else {
#pragma unroll 8
        for (int s = 0; s < C::DK / 4; ++s) {
            const int kk = 4 * s + g4;
            if constexpr (PART == 0) {
                mt = mma4(B.DH[j][kk], B.NK[j][kk], mt);
                mc = mma4(B.NK[j][kk], B.DH[j][kk], mc);
            } else {
                pt = mma4(B.DH[j][kk], B.QH[j][kk], pt);
            }
        }
    }
    // P row j (lower triangle including the diagonal); sweep: row j of P^T,
    // stored as [4 hi | 4 lo] per group of four tokens
    if constexpr (PART == 1) {
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            pv[e] = (C::BWD ? j <= 4 * g4 + e : 4 * g4 + e <= j) ? pt[e] : 0.f;
        if constexpr (C::BWD) {
            bf16x4 h, l;
            split4(f32x4{pv[0], pv[1], pv[2], pv[3]}, ne, h, l);
            *reinterpret_cast<bf16x8 *>(&B.PH[j][8 * g4]) = cat(h, l);
        } else if constexpr (BF) {
            bf16x4 h, l;
            split4(f32x4{pv[0], pv[1], pv[2], pv[3]}, ne, h, l);
            *reinterpret_cast<bf16x8 *>(&B.PH[j][8 * g4]) = cat(h, h);
            *reinterpret_cast<bf16x8 *>(&B.PL[j][8 * g4]) = cat(l, l);
        } else {
            *reinterpret_cast<OT4 *>(&B.PH[j][4 * g4]) = OT4{pv[0], pv[1], pv[2], pv[3]};
        }
        return;
    }
    // A[t][s] = beta_t M[t][s] (s < t), in D layout (a) and transposed (at)
    const float bj = B.BETA[j];
    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&B.BETA[4 * g4]);
    float skj = 1.f;
    f32x4 sk4 = {1.f, 1.f, 1.f, 1.f};
    if constexpr (C::GATED) {
        // L2 scales from the builders' partial sums: k_t = k~_t / |k~_t|
        // (and q alike) enter A as beta_t s_t s_s M~[t][s], T as
        // Diag(s_k) T, and the consumer's products as row scales
        float nq = 0.f, nk = 0.f;
        f32x4 nk4 = {0.f, 0.f, 0.f, 0.f};
        constexpr int NP = C::AUX ? 1 : C::NBW;      // partial sums per token
#pragma unroll
        for (int w = 0; w < NP; ++w) {
            nq += B.NRM[0][w][j];
            nk += B.NRM[1][w][j];
            nk4 += *reinterpret_cast<const f32x4 *>(&B.NRM[1][w][4 * g4]);
        }
        skj = __builtin_amdgcn_rsqf(nk + 1e-6f);
#pragma unroll
        for (int e = 0; e < 4; ++e) sk4[e] = __builtin_amdgcn_rsqf(nk4[e] + 1e-6f);
        if (g4 == 0) {
            B.SQ[j] = __builtin_amdgcn_rsqf(nq + 1e-6f);
            B.SK[j] = skj;
        }
    }
    // beta_t s_t s_s (s = 1 without the gated prologue)
    const float bsj = bj * skj;
    const f32x4 bs4 = b4 * sk4;
    f32x4 a, at, id;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * g4 + e;
        a[e] = (r > j) ? -bs4[e] * mc[e] * skj : 0.f;     // A[r][j]
        at[e] = (r < j) ? -bsj * mt[e] * sk4[e] : 0.f;    // A[j][r]
        id[e] = (r == j) ? 1.f : 0.f;
    }
    const Tile<BF> tA = to_tile<BF>(a), tAT = to_tile<BF>(at);
    const f32x4 a2 = prod<BF>(tAT, tA);             // A^2
    const f32x4 a2t = prod<BF>(tA, tAT);            // (A^2)^T
    const Tile<BF> tA2 = to_tile<BF>(a2), tA2T = to_tile<BF>(a2t);
    const f32x4 a4 = prod<BF>(tA2T, tA2);           // A^4
    const f32x4 a4t = prod<BF>(tA2, tA2T);          // (A^4)^T
    if constexpr (C::BWD) {
        // the same factors in the other orientation: lane (j, g4) ends with
        // column j of (I + A)^{-1}, rows 4 g4 .. 4 g4 + 3, so that
        // T^T[j][4 g4 + e] = beta_j (I + A)^{-1}[4 g4 + e][j]
        const f32x4 y1 = id - a + a2 - prod<BF>(tA2T, tA);     // (I - A)(I + A^2)
        const Tile<BF> tA4 = to_tile<BF>(a4), tA4T = to_tile<BF>(a4t);
        const f32x4 a8t = prod<BF>(tA4, tA4T);                  // (A^8)^T
        const Tile<BF> tY1 = to_tile<BF>(y1);
        const f32x4 y2 = y1 + prod<BF>(tA4T, tY1);              // (I + A^4) Y1
        const Tile<BF> tA8T = to_tile<BF>(a8t), tY2 = to_tile<BF>(y2);
        const f32x4 inv = y2 + prod<BF>(tA8T, tY2);             // (I + A^8) Y2
        if constexpr (C::CHUNK) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                B.MI[4 * g4 + e][j] = inv[e];
                B.KK[4 * g4 + e][j] = -mc[e];      // (KE Kd^T)[4 g4 + e][j]
            }
        }
        const f32x4 tv = inv * bj;
        bf16x4 h, l;
        split4(tv, ne, h, l);
        *reinterpret_cast<bf16x8 *>(&B.TH[j][8 * g4]) = cat(h, h);
        *reinterpret_cast<bf16x8 *>(&B.TL[j][8 * g4]) = cat(l, l);
        return;
    }
    // Y1^T = ((I - A)(I + A^2))^T = I - A^T + (A^2)^T - (A^2)^T A^T
    const f32x4 y1t = id - at + a2t - prod<BF>(tA2, tAT);
    const Tile<BF> tA4 = to_tile<BF>(a4), tA4T = to_tile<BF>(a4t);
    const f32x4 a8 = prod<BF>(tA4T, tA4);           // A^8
    // Y2^T = (Y1 (I + A^4))^T = Y1^T + (A^4)^T Y1^T
    const Tile<BF> tY1T = to_tile<BF>(y1t);
    const f32x4 y2t = y1t + prod<BF>(tA4, tY1T);
    // (I + A)^{-T} = Y2^T + (A^8)^T Y2^T: lane (j, g4) holds row j of the
    // inverse, columns 4 g4 .. 4 g4 + 3
    const Tile<BF> tA8 = to_tile<BF>(a8), tY2T = to_tile<BF>(y2t);
    const f32x4 tinv = y2t + prod<BF>(tA8, tY2T);
    // T = (I + A)^{-1} Diag(beta): column 4 g4 + e scaled by beta_{4 g4 + e}
    f32x4 tv = tinv * b4;
    if constexpr (C::GATED) tv *= skj;     // Diag(s_k) T
    if constexpr (BF) {
        bf16x4 h, l;
        split4(tv, ne, h, l);
        *reinterpret_cast<bf16x8 *>(&B.TH[j][8 * g4]) = cat(h, h);
        *reinterpret_cast<bf16x8 *>(&B.TL[j][8 * g4]) = cat(l, l);
    } else {
        *reinterpret_cast<OT4 *>(&B.TH[j][4 * g4]) = OT4{tv[0], tv[1], tv[2], tv[3]};
    }
}

// ---------------------------------------------------------------------------
// Longest sequences first.  The sequences of a packed batch can differ in
// length by orders of magnitude, and workgroups start in index order; a long
// sequence whose workgroups start late then sets the end of the launch.
// Dealing the sequences out longest first (ties by index) leaves the short
// ones for the tail.  The device holds cu_seqlens, so every wave ranks the
// sequences itself: lane l scores candidates l and l + 64, and the rank-r
// sequence is the one candidate whose score is r (a permutation, whatever
// the lengths).  Cost: n_seqs steps per wave, so only up to kLptMaxSeqs.
// ---------------------------------------------------------------------------
constexpr int kLptMaxSeqs = 128;
__device__ __forceinline__ int seq_of_rank(const int32_t *__restrict__ cu, int n_seqs, int r,
                                           int lane)
{
    auto len = [&](int s) -> int {
        if (s >= n_seqs) return -1;
        const int d = cu[s + 1] - cu[s];
        return d < 0 ? 0 : d;
    };
    const int s0 = lane, s1 = lane + 64;
    const int L0 = len(s0), L1 = len(s1);
    int k0 = 0, k1 = 0;                  // sequences ahead of s0 and s1
    for (int t = 0; t < n_seqs; ++t) {
        const int Lt = __builtin_amdgcn_readlane(t < 64 ? L0 : L1, t & 63);
        k0 += (Lt > L0 || (Lt == L0 && t < s0)) ? 1 : 0;
        k1 += (Lt > L1 || (Lt == L1 && t < s1)) ? 1 : 0;
    }
    const uint64_t m0 = __ballot(L0 >= 0 && k0 == r);
    const uint64_t m1 = __ballot(L1 >= 0 && k1 == r);
    return m0 ? __ffsll((unsigned long long)m0) - 1 : 64 + __ffsll((unsigned long long)m1) - 1;
}

// ---------------------------------------------------------------------------
// auxiliary waves (Cfg::AUX): the value block of a chunk (v, or dO in the
// sweep) and, in the forward, the Kd^T rows.  Aux thread a (0 .. 127) moves
// columns 2 (a % (BV / 2)) and the next one, tokens 4 (a / (BV / 2)) .. + 3,
// and writes the Kd^T row of channel a.
// ---------------------------------------------------------------------------
struct AuxV {
    uint32_t w[4];                       // 4 tokens x 2 bf16 columns
};
template <class C, typename TI>
__device__ __forceinline__ void aux_load_v(AuxV &x, const TI *__restrict__ v, int64_t tok_base,
                                           int ntok, int H, int h, int DV, int col_base, int a)
{
    static_assert(C::BV == 64 && C::DK == 128 && C::BF, "aux mapping");
    constexpr int CP = C::BV / 2;
    const int cp = a % CP, tq = a / CP;
    const int rowv = H * DV;
    const rsrc_t rv = make_rsrc(v + tok_base * rowv, ntok * rowv * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) x.w[i] = bload32(rv, ((4 * tq + i) * rowv + h * DV + col_base + 2 * cp) * 2);
}
template <class C>
__device__ __forceinline__ void aux_write_v(Buf<C> &B, const AuxV &x, int a)
{
    constexpr int CP = C::BV / 2;
    const int cp = a % CP, tq = a / CP;
    // column 2 cp takes the low halves of the four token words, 2 cp + 1 the high
    const uint32_t lo01 = __builtin_amdgcn_perm(x.w[1], x.w[0], 0x05040100u);
    const uint32_t lo23 = __builtin_amdgcn_perm(x.w[3], x.w[2], 0x05040100u);
    const uint32_t hi01 = __builtin_amdgcn_perm(x.w[1], x.w[0], 0x07060302u);
    const uint32_t hi23 = __builtin_amdgcn_perm(x.w[3], x.w[2], 0x07060302u);
    *reinterpret_cast<u32x2 *>(&B.VT[2 * cp][4 * tq]) = u32x2{lo01, lo23};
    *reinterpret_cast<u32x2 *>(&B.VT[2 * cp + 1][4 * tq]) = u32x2{hi01, hi23};
}
// gated prologue: |q|^2 and |k|^2 of each token.  Aux thread a takes
// token a / 8 and channels 16 (a % 8) .. + 15 of q and k (two 16-byte
// loads each); the 8 threads of a token sum with lane butterflies
struct AuxQK {
    u32x4 q[2], k[2];
};
template <class C, typename TI>
__device__ __forceinline__ void aux_load_qk(AuxQK &x, const TI *__restrict__ q,
                                            const TI *__restrict__ k, int64_t tok_base, int ntok,
                                            int H, int h, int a)
{
    const int rowk = H * C::DK;
    const rsrc_t rq = make_rsrc(q + tok_base * rowk, ntok * rowk * 2);
    const rsrc_t rk = make_rsrc(k + tok_base * rowk, ntok * rowk * 2);
    const int off = ((a >> 3) * rowk + h * C::DK + 16 * (a & 7)) * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        x.q[i] = bload128(rq, off + 16 * i);
        x.k[i] = bload128(rk, off + 16 * i);
    }
}
template <class C>
__device__ __forceinline__ void aux_norms(Buf<C> &B, const AuxQK &x, int a)
{
    float nq = 0.f, nk = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float q0 = __uint_as_float(x.q[i][e] << 16), q1 = __uint_as_float(x.q[i][e] & 0xffff0000u);
            const float k0 = __uint_as_float(x.k[i][e] << 16), k1 = __uint_as_float(x.k[i][e] & 0xffff0000u);
            nq = __builtin_fmaf(q0, q0, __builtin_fmaf(q1, q1, nq));
            nk = __builtin_fmaf(k0, k0, __builtin_fmaf(k1, k1, nk));
        }
    nq = group_sum<8>(nq);
    nk = group_sum<8>(nk);
    if ((a & 7) == 0) {
        B.NRM[0][0][a >> 3] = nq;
        B.NRM[1][0][a >> 3] = nk;
    }
}
template <class C>
__device__ __forceinline__ void aux_kh(Buf<C> &B, int a)
{
    const int kc = kpos<C>(a);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        bf16x8 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[i] = B.DH[4 * g + i][kc];
            r[4 + i] = B.DL[4 * g + i][kc];
        }
        *reinterpret_cast<bf16x8 *>(&B.KH[a][8 * g]) = r;
    }
}

}  // namespace kda
