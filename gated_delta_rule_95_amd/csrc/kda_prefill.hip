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
template <typename TI, int DK_, int NW_, int NBUF_, bool GATED_ = false>
struct Cfg {
    static constexpr bool BF = std::is_same<TI, bf16>::value;
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
    static constexpr int NT = (NW + NBW + 2) * WAVE;   // consumers, builders, 2 helpers
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
    using OT = typename C::OT;
    OT NK[16][C::LDK];                   // -KE                  [token][channel]
    OT QH[16][C::LDK];                   // QE hi
    OT QL[C::LO ? 16 : 1][C::LDK];       // QE lo
    OT DH[16][C::LDK];                   // Kd hi                [token][channel]
    OT DL[C::LO ? 16 : 1][C::LDK];       // Kd lo
    OT KH[C::DK][C::LDT];                // Kd^T                 [channel][token]
    OT TH[16][C::LDP];                   // T (hi)               [token r][token i]
    OT TL[C::LO ? 16 : 1][C::LDP];       // T lo
    OT PH[16][C::LDP];                   // P (hi)
    OT PL[C::LO ? 16 : 1][C::LDP];       // P lo
    OT VT[C::BV][C::LVT];                // value block, transposed  [column][token]
    float DEC[C::DK];                    // e^{Gc_16} per channel
    float BETA[16];
    // gated prologue: per builder wave, the partial sums of q^2 and k^2 of
    // each token over its channels; then the scales 1 / |q|, 1 / |k|
    float NRM[C::GATED ? 2 : 1][C::GATED ? C::NBW : 1][16];
    float SQ[C::GATED ? 16 : 1], SK[C::GATED ? 16 : 1];
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
    if constexpr (C::GATED) {
        // partial |q|^2 and |k|^2 of this lane's tokens over the wave's
        // channels: sum the channel pairs of the CPW lanes of a token group
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
#pragma unroll
    for (int t = 0; t < TPG; ++t) {
        const int tok = tok0 + t;
        const float d0 = G0[t] + o0, d1 = G1[t] + o1;                 // >= 0 (log2)
        const float e0 = fast_exp2(d0), e1 = fast_exp2(d1);           // E
        const float f0 = fast_exp2(-d0), f1 = fast_exp2(-d1);         // 1 / E
        const float ka = elem<C>(r.k[t], 0), kb = elem<C>(r.k[t], 1);
        const float qa = elem<C>(r.q[t], 0), qb = elem<C>(r.q[t], 1);
        qk[t] = f32x4{qa * e0, qb * e1, ka * f0, kb * f1};
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
                const bf16x2 vh = __builtin_bit_cast(bf16x2, dh), vl = __builtin_bit_cast(bf16x2, dl);
                kdh0[t + u] = vh[0]; kdh1[t + u] = vh[1]; kdl0[t + u] = vl[0]; kdl1[t + u] = vl[1];
            }
        }
    }
    // Kd^T rows: this lane's TPG consecutive tokens of channels ch, ch + 1
    if constexpr (C::BF) {
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
        if (C::all_v(tid)) {
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
                    pt = mma32(dh, qh, pt);
                    pt = mma32(dl, qh, pt);
                    pt = mma32(dh, ql, pt);
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
    // P row j (lower triangle including the diagonal)
    if constexpr (PART == 1) {
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = (4 * g4 + e <= j) ? pt[e] : 0.f;
        if constexpr (BF) {
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
#pragma unroll
        for (int w = 0; w < C::NBW; ++w) {
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
// the D layout: lane (j, g4) holds O[token j][columns 4 g4 .. 4 g4 + 3]
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ f32x4 consume(const Buf<C> &B, f32x4 (&S)[C::DK / 16],
                                         const Ahead<C> &ah, int wave, int lane)
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
                // stored positions 32 s + 8 g4 .. + 7 hold exactly these channels
                const int kk = 32 * s + 8 * g4;
                const bf16x8 nk = s == 0 ? ah.nk : ld8b(&B.NK[j][kk]);
                const bf16x8 qh = s == 0 ? ah.qh : ld8b(&B.QH[j][kk]);
                const bf16x8 ql = s == 0 ? ah.ql : ld8b(&B.QL[j][kk]);
                x = mma32(nk, sh, x);
                x = mma32(nk, sl, x);
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
    // every chunk c of sequence n goes to slot bos / 16 + n + c of ckpt, as
    // [slot][H][d_v / 16][d_k / 16][64][4] floats: per 16 x 16 tile (key rows
    // 16 t .., value columns 16 cb ..), lane j + 16 g of the tile holds rows
    // 16 t + 4 g .. + 3 of column 16 cb + j; o is not written
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
    // helper waves sit on SIMDs 0 and 1.  Every role runs its own loop; the
    // role is wave-uniform.
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
        // checkpoint tiles of this wave's 16 columns, chunk 0 of the sequence
        f32x4 *ck = nullptr;
        if constexpr (CKPT)
            ck = reinterpret_cast<f32x4 *>(p.ckpt + ((bos / 16 + n) * H + h) * (int64_t)(DK * DV)) +
                 ((col_base / 16 + wave) * (DK / 16)) * WAVE + lane;
#pragma unroll 1
        for (int c = 0; c < nch; ++c) {
            store_o(c - 1);
            if constexpr (CKPT) {
#pragma unroll
                for (int t = 0; t < DK / 16; ++t)
                    ck[(int64_t)c * H * (DK * DV / 4) + t * WAVE] = S[t];
            }
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
// of one token.  One workgroup per (chain, segment, 256 tokens); E_s^T is
// staged in LDS as bf16 hi and lo rows.
// ---------------------------------------------------------------------------
template <typename TO, int DK, int DV>
__global__ __launch_bounds__(256) void kda_seg_correct_kernel(
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
    const int tb = 256 * tile;
    if (tb >= segT) return;
    const int ntile = segT - tb < 256 ? segT - tb : 256;

    // E_s^T as hi/lo bf16: thread takes rows r, r + 1 of one column c
    const float *E = entry + ((int64_t)chain * (nseg - 1) + seg - 1) * DK * DV;
    for (int e = threadIdx.x; e < DK * DV / 2; e += 256) {
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
    for (int it = 0; it < 4; ++it) {
        const int tt = 64 * it + 16 * wave;
        if (tt >= ntile) break;
        const int nt = ntile - tt < 16 ? ntile - tt : 16;
        const rsrc_t rr = make_rsrc(rq + (aug0 + tt) * H * DK, nt * H * DK * 4);
        const rsrc_t r0 = make_rsrc(o0 + (aug0 + tt) * H * DV, nt * H * DV * 4);
        const rsrc_t ro = make_rsrc(o + (tok0 + tt) * H * DV, nt * H * DV * (int)sizeof(TO));
        // B = R^T: lane (token nn, kg) holds R[nn][32 s + 8 kg .. + 7]
        bf16x8 rh[DK / 32], rl[DK / 32];
#pragma unroll
        for (int s2 = 0; s2 < DK / 32; ++s2) {
            const int off = ((nn * H + h) * DK + 32 * s2 + 8 * kg) * 4;
            const f32x4 a = __builtin_bit_cast(f32x4, bload128(rr, off));
            const f32x4 b = __builtin_bit_cast(f32x4, bload128(rr, off + 16));
            const u32x4 hw = {pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(b[0], b[1]),
                              pack2(b[2], b[3])};
            rh[s2] = __builtin_bit_cast(bf16x8, hw);
            f32x4 ra, rb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra[i] = a[i] - (float)rh[s2][i];
                rb[i] = b[i] - (float)rh[s2][4 + i];
            }
            const u32x4 lw = {pack2(ra[0], ra[1]), pack2(ra[2], ra[3]), pack2(rb[0], rb[1]),
                              pack2(rb[2], rb[3])};
            rl[s2] = __builtin_bit_cast(bf16x8, lw);
        }
#pragma unroll 2
        for (int ct = 0; ct < DV / 16; ++ct) {
            // lane (token nn, kg) accumulates O[nn][16 ct + 4 kg .. + 3]
            const int ocol = (nn * H + h) * DV + 16 * ct + 4 * kg;
            f32x4 acc = __builtin_bit_cast(f32x4, bload128(r0, ocol * 4));
#pragma unroll
            for (int s2 = 0; s2 < DK / 32; ++s2) {
                const bf16x8 ah = ld8b(&EH[16 * ct + nn][32 * s2 + 8 * kg]);
                const bf16x8 al = ld8b(&EL[16 * ct + nn][32 * s2 + 8 * kg]);
                acc = mma32(ah, rh[s2], acc);
                acc = mma32(al, rh[s2], acc);
                acc = mma32(ah, rl[s2], acc);
            }
            bstore4(ro, ocol * (int)sizeof(TO), acc, TO{});
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
        const int tiles = (pl.lenS + 255) / 256;
        const int64_t g2 = chains * (pl.nseg - 1) * tiles;
        hipLaunchKernelGGL((kda_seg_correct_kernel<TO, DK, DV>), dim3((unsigned)g2), dim3(256), 0,
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
