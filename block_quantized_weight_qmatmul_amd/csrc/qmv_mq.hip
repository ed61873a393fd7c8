// qmv_mq.hip — Q4_0 / Q8_0 products with 2..16 activation rows on the matrix
// cores of gfx950 (v_mfma_f32_16x16x32_bf16): the batched-verify shape of the
// hf2q pages (several tokens through one `dispatch_qmatmul`, m > 1), and each
// 16-row block of a prefill. One launch per call; the kernel needs no memory
// beyond the caller's inputs and outputs, so a call can be captured into a
// HIP graph as it is.
//
// The product per block of 32 weights: Y[m, n] += d[n] * sum_k c[n, k] X[m, k]
// with c the integer code (Q4_0: code - 8, Q8_0: the int8 code). One MFMA
// multiplies 16 activation rows (A) by one block of 16 weight rows (B) and
// returns the 16 x 16 block sums; the fp16 block scale d is applied in fp32
// to them and they are added to the running sums.
//
// Operands:
//  * B: the codes as bf16, exact (Q4_0: (code - 8) / 16 from
//    v_cvt_off_f32_i4 on code ^ 8, the 1/16 undone on output; Q8_0: the int8
//    code). Lanes load whole 36-byte (Q4_0) or 68-byte (Q8_0) block pairs of
//    their weight row; two 4 x 4 transposes across the wave's 16-lane rows
//    hand every lane its MFMA slice of each of the step's 8 blocks.
//  * A: each fp32 activation x split into two bf16, x = hi + lo + r with
//    hi = x truncated to bf16 (never rounded up, so finite for every finite
//    x) and lo = bf16(x - hi) of the exact difference: |x - hi| < 2^-7 |x|,
//    so |r| < 2^-16 |x|. bf16 keeps the fp32 exponent, so no activation row
//    needs scaling and no value can fall out of range. An infinity or NaN
//    keeps its value in hi, lo = 0. Each workgroup converts the activation
//    columns of the step it is about to use into LDS, one step ahead, from
//    registers loaded one step before that.
//
// Work split: a tile is 16 weight rows. A workgroup owns WAVES / KS tiles;
// the KS waves of a tile take its steps (8 blocks = 256 columns) in turn,
// so all waves of the workgroup work on the same KS consecutive steps
// (one "round") at a time, and their partial sums are added in a fixed order
// through LDS at the end (no atomics: bitwise reproducible). Each wave keeps
// the weight loads of its next round in flight (the launch shapes split every
// tile over two or four waves, so that the kernel fits in 96-116 registers and
// a compute unit runs 8-14 waves).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qmv.h"
#include "qmv_internal.h"

namespace qmvi {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4a_t __attribute__((ext_vector_type(4), aligned(4)));

constexpr int MQ_STEP_BYTES = 8 * 2048;  // A operands of one step: 8 blocks x {hi, lo} x 4 slices x 16 rows x 16 B

template <int QT>
struct MqFmt;
// Q4_0: a pair of blocks is 36 bytes (9 dwords). The MFMA slice G of a block
// is qs dword G: its low nibbles are elements 4G..4G+3, its high nibbles
// elements 16+4G..16+4G+3, in that order.
template <>
struct MqFmt<QMV_Q4_0> {
    static constexpr int DW = 9;
    static constexpr float OUT_SCALE = 16.f;
    __host__ __device__ static constexpr int xoff(int G, int h) { return 16 * h + 4 * G; }
};
// Q8_0: a pair is 68 bytes (17 dwords). Slice G of a block = codes 8G..8G+7.
template <>
struct MqFmt<QMV_Q8_0> {
    static constexpr int DW = 17;
    static constexpr float OUT_SCALE = 1.f;
    __host__ __device__ static constexpr int xoff(int G, int h) { return 8 * G + 4 * h; }
};

// Two fp32 whose low 16 bits are zero (exact bf16 values) as a bf16 pair.
__device__ __forceinline__ uint32_t pack_bf16_exact(float a, float b) {
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a), 0x07060302u);
}

// Q4_0 slice: one qs dword -> 8 bf16 (code - 8) / 16, elements
// 4G, 4G+1, 4G+2, 4G+3, 16+4G, 16+4G+1, 16+4G+2, 16+4G+3.
__device__ __forceinline__ bf16x8_t dec_q4(uint32_t q) {
    const uint32_t u = q ^ 0x88888888u, u4 = hi_nibbles(u);
    const uint32_t p0 = pack_bf16_exact(nib<0>(u), nib<1>(u));
    const uint32_t p1 = pack_bf16_exact(nib<2>(u), nib<3>(u));
    const uint32_t p2 = pack_bf16_exact(nib<0>(u4), nib<1>(u4));
    const uint32_t p3 = pack_bf16_exact(nib<2>(u4), nib<3>(u4));
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x8_t, (u32x4v){p0, p1, p2, p3});
}

// Q8_0 slice: two code dwords -> 8 bf16 int8 codes, in byte order.
__device__ __forceinline__ bf16x8_t dec_q8(uint32_t a, uint32_t b) {
    auto sb = [](uint32_t w, int k) { return (float)(int8_t)(w >> (8 * k)); };
    const uint32_t p0 = pack_bf16_exact(sb(a, 0), sb(a, 1));
    const uint32_t p1 = pack_bf16_exact(sb(a, 2), sb(a, 3));
    const uint32_t p2 = pack_bf16_exact(sb(b, 0), sb(b, 1));
    const uint32_t p3 = pack_bf16_exact(sb(b, 2), sb(b, 3));
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x8_t, (u32x4v){p0, p1, p2, p3});
}

// Eight activations -> A operand record: hi (4 dwords) and lo (4 dwords).
constexpr float BF16_MAX = 0x1.fcp127f;  // largest finite bf16 (0x7F7F)
__device__ __forceinline__ void split_bf16(const float (&v)[8], uint32_t (&hw)[4], uint32_t (&lw)[4]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    // All eight finite and below the largest bf16: the common case, taken by
    // the whole wave or not at all.
    bool ok = true;
#pragma unroll
    for (int e = 0; e < 8; ++e) ok = ok && fabsf(v[e]) < BF16_MAX;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!ok) == 0, 1)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bf16x2 h = {(__bf16)v[2 * k], (__bf16)v[2 * k + 1]};
            const uint32_t hb = __builtin_bit_cast(uint32_t, h);
            const float r0 = v[2 * k] - __builtin_bit_cast(float, hb << 16);
            const float r1 = v[2 * k + 1] - __builtin_bit_cast(float, hb & 0xFFFF0000u);
            const bf16x2 l = {(__bf16)r0, (__bf16)r1};
            hw[k] = hb;
            lw[k] = __builtin_bit_cast(uint32_t, l);
        }
    } else {
        // per element: as above below the largest bf16; a larger finite x
        // takes hi = x rounded toward zero (finite) and lo = bf16(x - hi); an
        // infinity keeps its value in hi and a NaN stays a NaN, with lo = 0
        uint16_t h[8], l[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = v[e];
            const uint32_t xb = __builtin_bit_cast(uint32_t, x);
            if (fabsf(x) < BF16_MAX) {
                const __bf16 hx = (__bf16)x;
                h[e] = __builtin_bit_cast(uint16_t, hx);
                l[e] = __builtin_bit_cast(uint16_t, (__bf16)(x - (float)hx));
            } else if (fabsf(x) <= 0x1.fffffep127f) {
                h[e] = (uint16_t)(xb >> 16);
                l[e] = __builtin_bit_cast(uint16_t, (__bf16)(x - __builtin_bit_cast(float, xb & 0xFFFF0000u)));
            } else {
                h[e] = (uint16_t)((xb >> 16) | (x != x ? 0x0040u : 0u));
                l[e] = 0;
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            hw[k] = h[2 * k] | ((uint32_t)h[2 * k + 1] << 16);
            lw[k] = l[2 * k] | ((uint32_t)l[2 * k + 1] << 16);
        }
    }
}

// Eight activations -> A operand record with hi = x truncated to bf16 (never
// rounds up, so every finite x has a finite hi) and lo = bf16(x - hi) of the
// exact difference. Infinities and NaNs, the only inputs whose difference is
// a NaN, take split_bf16's per-element rules instead; that test is one wave
// ballot per pair, combined in scalar registers.
__device__ __forceinline__ void split_bf16_trunc(const float (&v)[8], uint32_t (&hw)[4], uint32_t (&lw)[4]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint64_t bad = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t a = __builtin_bit_cast(uint32_t, v[2 * k]), b = __builtin_bit_cast(uint32_t, v[2 * k + 1]);
        const float r0 = v[2 * k] - __builtin_bit_cast(float, a & 0xFFFF0000u);
        const float r1 = v[2 * k + 1] - __builtin_bit_cast(float, b & 0xFFFF0000u);
        bad |= __builtin_amdgcn_ballot_w64(__builtin_isunordered(r0, r1));
        hw[k] = __builtin_amdgcn_perm(b, a, 0x07060302u);
        const bf16x2 l = {(__bf16)r0, (__bf16)r1};
        lw[k] = __builtin_bit_cast(uint32_t, l);
    }
    if (__builtin_expect(bad != 0, 0)) split_bf16(v, hw, lw);
}

// ---------------------------------------------------------------------------
// The kernel. grid.x = (tile groups) * mblocks, the 16-row block of X / Y
// fastest, so the workgroups that read one weight tile run side by side.
// ---------------------------------------------------------------------------
template <int QT, int WAVES, int KS, int WD = 4>
__global__ __launch_bounds__(WAVES * 64) void k_mq(const uint8_t* __restrict__ W, size_t ldw,
                                                   const float* __restrict__ X, size_t ldx, float* __restrict__ Y,
                                                   size_t ldy, int M, int N, int K, int mblocks, int seg_rounds,
                                                   float* __restrict__ part) {
    using F = MqFmt<QT>;
    constexpr int DW = F::DW, PB = 4 * DW;
    constexpr int NT = WAVES * 64;
    constexpr int TWG = WAVES / KS;            // tiles per workgroup
    constexpr int REC = 512 * KS;              // A records (16 B hi + 16 B lo) per round
    constexpr int RPT = (REC + NT - 1) / NT;   // records per thread
    // activation register sets in flight (fewer with the 68-byte Q8_0 pairs)
    constexpr int XS = WD == 1 ? 1 : WD == 2 ? 2 : ((QT == QMV_Q8_0 || WAVES % 4 != 0) && RPT <= 2) ? 2 : RPT <= 4 ? 4 : 2;
    static_assert(WD % XS == 0, "activation sets must divide the weight depth");
    constexpr int ROUND_BYTES = KS * MQ_STEP_BYTES;
    extern __shared__ __align__(16) uint8_t smem[];  // A operands of two rounds

    const int mb = blockIdx.x % mblocks;
    const long grp = blockIdx.x / mblocks;
    X += (size_t)mb * 16 * ldx;
    Y += (size_t)mb * 16 * ldy;
    const int Mb = M - mb * 16 < 16 ? M - mb * 16 : 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = lane >> 4, j = lane & 15;
    const int tw = wave / KS, sp = wave % KS;
    const long row0 = (grp * TWG + tw) * 16;
    const int P = K >> 6;             // block pairs per row
    const int S = (P + 3) >> 2;       // steps per row
    const int nb = K >> 5;            // blocks per row
    const int rounds = (S + KS - 1) / KS;
    // K segment blockIdx.y: rounds r0 .. r0 + nr - 1 (all of them with one segment)
    const int r0 = blockIdx.y * seg_rounds;
    const int nr = (rounds - r0 < seg_rounds ? rounds - r0 : seg_rounds);
    long wr = row0 + j;
    wr = wr < N ? wr : N - 1;
    const uint8_t* __restrict__ wrow = W + wr * ldw;

    // ---- weights: the pair 4t + G of this lane's row, t = this wave's step
    // of round r0 + r (r counts the rounds of this workgroup's K segment)
    auto issue = [&](int r, uint32_t (&b)[DW]) __attribute__((always_inline)) {
        int q = ((r0 + r) * KS + sp) * 4 + G;
        q = q < P ? q : P - 1;  // past the row end: the last pair again (not used)
        load_pair<DW>(wrow + (size_t)q * PB, b);
    };
    // ---- activations. Record rho of a round = (step in round, block, slice
    // G, row m) with rho = tid + i * NT: every record of a thread has the
    // thread's own (G, m) = (lane % 4, lane / 4) and block (wave + i * WAVES)
    // of the round. Every lane loads from a valid address (rows past M and
    // blocks past K clamped), so the loads carry no branch and the wait before
    // their use counts exactly the loads issued after them; such records are
    // stored as zeros.
    // (the thread loads slice xg of row xj: the four lanes of a quad read one
    // row's 64 contiguous bytes; the record goes to operand slot (xg, xj))
    const int xj = lane >> 2, xg = lane & 3;
    const bool mok = xj < Mb;
    const float* __restrict__ xb = X + (size_t)(mok ? xj : Mb - 1) * ldx + F::xoff(xg, 0);
    constexpr int XD = F::xoff(0, 1) - F::xoff(0, 0);  // second 4-float run of a record
    auto fetch_x = [&](int r, f32x4a_t (&xr)[RPT][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            int blk = (r0 + r) * 8 * KS + wave + i * WAVES;
            blk = blk < nb ? blk : nb - 1;
            const float* src = xb + (size_t)blk * 32;
            xr[i][0] = *reinterpret_cast<const f32x4a_t*>(src);
            xr[i][1] = *reinterpret_cast<const f32x4a_t*>(src + XD);
        }
    };
    auto put_x = [&](int r, int buf, const f32x4a_t (&xr)[RPT][2]) __attribute__((always_inline)) {
        // operand slot (G, m) of a block sits at G * 256 + ((m + 4G) % 16) * 16,
        // which spreads the stores of a quarter wave (four rows, four slices
        // each) over the row while a lane row G of the reads still covers one
        // contiguous 256-byte row (measured about 1% faster than slot 16G + m)
        uint8_t* base = smem + buf * ROUND_BYTES + wave * 2048 + xg * 256 + ((xj + 4 * xg) & 15) * 16;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            if ((8 * KS) % WAVES != 0 && wave + i * WAVES >= 8 * KS) continue;  // past the round's blocks
            uint8_t* rec = base + i * WAVES * 2048;
            u32x4 hi = {0u, 0u, 0u, 0u}, lo = hi;
            if (mok && (r0 + r) * 8 * KS + wave + i * WAVES < nb) {
                const float v[8] = {xr[i][0].x, xr[i][0].y, xr[i][0].z, xr[i][0].w,
                                    xr[i][1].x, xr[i][1].y, xr[i][1].z, xr[i][1].w};
                uint32_t hw[4], lw[4];
                split_bf16_trunc(v, hw, lw);
                hi = (u32x4){hw[0], hw[1], hw[2], hw[3]};
                lo = (u32x4){lw[0], lw[1], lw[2], lw[3]};
            }
            *reinterpret_cast<u32x4*>(rec) = hi;
            *reinterpret_cast<u32x4*>(rec + 1024) = lo;
        }
    };

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // ---- one step: 8 blocks of the tile (2 per lane group, pair 4t + c for lane group c)
    auto compute = [&](int r, const uint32_t (&b)[DW]) __attribute__((always_inline)) {
        const int t = (r0 + r) * KS + sp;
        const bool valid = t * 4 + G < P;
        const uint8_t* xa = smem + (r & 1) * ROUND_BYTES + sp * MQ_STEP_BYTES + G * 256 + ((j + 4 * G) & 15) * 16;
        // both block scales of this lane's pair in one dword; zero past K
        uint32_t dd[4];
        const uint32_t dpk = valid ? ((b[0] & 0xFFFFu) | (QT == QMV_Q4_0 ? (b[4] & 0xFFFF0000u) : (b[8] & 0xFFFF0000u))) : 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) dd[c] = dpk;
        xpose4(dd);  // dd[c] = scales of lane group c's pair
        // B slices of the step's 8 blocks: slice of block 2c + R in bq_src(c, R)
        uint32_t v0[4], v1[4], w0[4], w1[4];
        if constexpr (QT == QMV_Q4_0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v0[u] = __builtin_amdgcn_alignbyte(b[u + 1], b[u], 2);
                v1[u] = b[5 + u];
            }
            xpose4(v0);  // v0[c] = qs dword G of the first block of pair c
            xpose4(v1);
        } else {
            // block 0 codes at bytes 2..33 (dwords 0..8, shifted by 2), block 1 at 36..67 (dwords 9..16)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v0[u] = __builtin_amdgcn_alignbyte(b[2 * u + 1], b[2 * u], 2);
                w0[u] = __builtin_amdgcn_alignbyte(b[2 * u + 2], b[2 * u + 1], 2);
                v1[u] = b[9 + 2 * u];
                w1[u] = b[10 + 2 * u];
            }
            xpose4(v0);  // v0[c] = code dword 2G of the first block of pair c
            xpose4(w0);  //          w0[c]: code dword 2G + 1
            xpose4(v1);
            xpose4(w1);
        }
        // A operands one block ahead of the one being multiplied
        bf16x8_t ah[2], al[2];
        ah[0] = *reinterpret_cast<const bf16x8_t*>(xa);
        al[0] = *reinterpret_cast<const bf16x8_t*>(xa + 1024);
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
            const int c = blk >> 1, R = blk & 1;
            if (blk + 1 < 8) {
                ah[(blk + 1) & 1] = *reinterpret_cast<const bf16x8_t*>(xa + (blk + 1) * 2048);
                al[(blk + 1) & 1] = *reinterpret_cast<const bf16x8_t*>(xa + (blk + 1) * 2048 + 1024);
            }
            bf16x8_t bq;
            if constexpr (QT == QMV_Q4_0)
                bq = dec_q4(R ? v1[c] : v0[c]);
            else
                bq = R ? dec_q8(v1[c], w1[c]) : dec_q8(v0[c], w0[c]);
            f32x4_t cc = {0.f, 0.f, 0.f, 0.f};
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[blk & 1], bq, cc, 0, 0, 0);
            cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[blk & 1], bq, cc, 0, 0, 0);
            const float d = R ? half_hi(dd[c]) : half_lo(dd[c]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = fmaf(d, cc[i], acc[i]);
        }
    };

    // ---- pipeline: weights WD rounds ahead; activations converted one
    // round ahead, from registers loaded XS rounds before that (XS register
    // sets, X(k) in set k % XS). Loads past the last round read valid
    // addresses and are not used, so that no load is conditional (a
    // conditional load makes the compiler wait for all loads).
    f32x4a_t xr[XS][RPT][2];
    uint32_t bw[WD][DW];
    fetch_x(0, xr[0]);  // before the weight loads: waiting for it leaves them in flight
#pragma unroll
    for (int k = 0; k < WD; ++k) issue(k, bw[k]);
    put_x(0, 0, xr[0]);
#pragma unroll
    for (int k = 1; k <= XS; ++k) fetch_x(k, xr[k % XS]);
    lds_barrier();
    // round r: its step, the weights of round r + WD, the activations of
    // round r + 1 into LDS and those of round r + 1 + XS into the freed set
    auto body = [&](int r, uint32_t (&bb)[DW], auto SET) __attribute__((always_inline)) {
        constexpr int xs = decltype(SET)::value;
        compute(r, bb);
        issue(r + WD, bb);
        put_x(r + 1, (r + 1) & 1, xr[xs]);
        fetch_x(r + 1 + XS, xr[xs]);
        lds_barrier();
        // rounds stay apart: no work of the next round is hoisted above the
        // barrier (it would only hold registers)
        __builtin_amdgcn_sched_barrier(0);
    };
    // Whole groups of WD rounds in the loop, the rest after it: every path
    // into the loop's first round then has the same loads in flight.
    int r = 0;
    for (; r + WD <= nr; r += WD)
        unroll<0, WD>([&](auto k) { body(r + k, bw[k], std::integral_constant<int, (k + 1) % XS>{}); });
    unroll<0, WD - 1>([&](auto k) {
        if (r + k < nr) body(r + k, bw[k], std::integral_constant<int, (k + 1) % XS>{});
    });

    // ---- the KS partial sums of a tile, added in order sp = 0, 1, ...
    // lane (G, j) holds activation rows 4G..4G+3 of weight row j
    if constexpr (KS > 1) {
        f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);  // [tile][sp - 1][lane]
        if (sp > 0) red[(tw * (KS - 1) + sp - 1) * 64 + lane] = acc;
        lds_barrier();
        if (sp > 0) return;
#pragma unroll
        for (int s = 1; s < KS; ++s) {
            const f32x4_t o = red[(tw * (KS - 1) + s - 1) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += o[i];
        }
    }
    const long row = row0 + j;
    if (row < N) {
        // with K segments: partial sums part[segment][m][n] (M rows of N), summed by k_mqred
        float* dst = part ? part + ((size_t)blockIdx.y * M + (size_t)mb * 16) * N + row : Y + row;
        const size_t ld = part ? (size_t)N : ldy;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * G + i;
            if (m < Mb) dst[(size_t)m * ld] = acc[i] * F::OUT_SCALE;
        }
    }
}

// Y[m, n] = the S partial sums part[s][m][n] added in segment order. Up to
// 16 partial sums are loaded at once (the addresses of those past S clamped
// to the last one, not added), so S <= 16 costs one memory latency.
__global__ __launch_bounds__(256) void k_mqred(const float* __restrict__ part, int S, int M, int N,
                                               float* __restrict__ Y, size_t ldy) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)M * N) return;
    const size_t mn = (size_t)M * N;
    const float* p = part + i;
    float t = 0.f;
    for (int s0 = 0; s0 < S; s0 += 16) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = p[(size_t)(s0 + k < S ? s0 + k : S - 1) * mn];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (s0 + k < S) t = s0 + k == 0 ? v[k] : t + v[k];
    }
    Y[(size_t)(i / N) * ldy + (size_t)(i % N)] = t;
}

// Launch plan: workgroup shape and K segments (S = 1: no segments, no workspace).
struct MqPlan {
    int waves, ks, S, seg_rounds;
    size_t ws_bytes;
};

// ws_cap: the most workspace bytes the call may use (0: none, scratch-free).
MqPlan plan_mq(int qtype, int M, int N, int K, size_t ws_cap) {
    const long tiles = ((long)N + 15) / 16;
    const long ncu = num_cus();
    const long mblocks = ((long)M + 15) / 16;
    const int steps = ((K >> 6) + 3) >> 2;
    MqPlan p{8, 1, 1, steps, 0};
    if (tiles * mblocks >= 4 * ncu) {
        // One wave per tile fills the chip. Seven tiles per workgroup,
        // each split over two waves that take alternate steps, with the
        // weights one round ahead (96 registers, so 14 waves fit a compute
        // unit; a streaming read with 7-8 waves per unit runs 10-15% slower
        // than with 16). N = 27648: 30.0 us, against 32.9 with one wave per
        // tile and weights four rounds ahead (Q4_0); Q8_0 44.0 against 45.8.
        p.waves = 14;
        p.ks = 2;
        return p;
    }
    // Few tiles. Without a workspace: two tiles per workgroup, each split over
    // four waves, every workgroup reading and converting all of X. With one:
    // four tiles per workgroup (each split over two waves) and K cut into
    // segments of whole rounds over grid.y, so that about one workgroup per
    // compute unit each reads and converts only its segment of X; the partial
    // sums go to the workspace and a second launch adds them in segment order
    // (M = 16, K = 5120, graph-timed: N = 5120 13.8 us with 3 segments,
    // N = 1024 8.6 us with 10).
    const long groups = ((tiles + 3) / 4) * mblocks;
    long S = (ncu + groups / 2) / groups;  // about one workgroup per compute unit
    S = S < steps ? S : steps;
    const size_t per_seg = (size_t)M * N * sizeof(float);
    if (ws_cap / per_seg < (size_t)S) S = (long)(ws_cap / per_seg);
    if (S < 2) {
        // two tiles per workgroup, each split over four waves (M = 16,
        // K = 5120: N = 5120 19.8 -> 14.7 us, N = 1024 19.4 -> 14.4 us
        // against two waves per tile)
        p.waves = 8;
        p.ks = 4;
        p.seg_rounds = (steps + 3) / 4;
        return p;
    }
    // each tile split over two waves (weights one round ahead): 8 waves a
    // workgroup instead of 4 (M = 16, K = 5120: N = 5120 15.6 -> 13.8 us,
    // N = 1024 9.1 -> 8.6 us)
    const int rds = (steps + 1) / 2;
    const int seg = (int)((rds + S - 1) / S);
    p.waves = 8;
    p.ks = 2;
    p.seg_rounds = seg;
    p.S = (rds + seg - 1) / seg;
    p.ws_bytes = (size_t)p.S * per_seg;
    return p;
}

template <int QT, int WAVES, int KS, int WD = 4>
int launch_mq_t(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
                int S, int seg_rounds, float* part, hipStream_t st) {
    constexpr int TWG = WAVES / KS;
    const long tiles = ((long)N + 15) / 16;
    const long groups = (tiles + TWG - 1) / TWG;
    const long mblocks = ((long)M + 15) / 16;
    if (groups * mblocks > 0x7FFFFFFF || S > 65535) return fail(QMV_EINVAL, "N too large");
    const size_t lds = (size_t)2 * KS * MQ_STEP_BYTES;
    hipLaunchKernelGGL((k_mq<QT, WAVES, KS, WD>), dim3((unsigned)(groups * mblocks), (unsigned)S), dim3(WAVES * 64), lds,
                       st, W, ldw, X, ldx, Y, ldy, M, N, K, (int)mblocks, seg_rounds, S > 1 ? part : nullptr);
    int rc = check_launch("qmv matrix-core kernel");
    if (rc == QMV_OK && S > 1) {
        const long n = (long)M * N;
        hipLaunchKernelGGL(k_mqred, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const float*)part, S, M, N, Y,
                           ldy);
        rc = check_launch("qmv matrix-core partial-sum launch");
    }
    return rc;
}

template <int QT>
int launch_mq_q(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
                const MqPlan& p, float* part, hipStream_t st) {
    const int S = p.S, sr = p.seg_rounds;
    if (p.waves == 14 && p.ks == 2) return launch_mq_t<QT, 14, 2, 1>(W, ldw, X, ldx, Y, ldy, M, N, K, S, sr, part, st);
    if (p.waves == 8 && p.ks == 2) return launch_mq_t<QT, 8, 2, 1>(W, ldw, X, ldx, Y, ldy, M, N, K, S, sr, part, st);
    if (p.waves == 8 && p.ks == 4) return launch_mq_t<QT, 8, 4, 1>(W, ldw, X, ldx, Y, ldy, M, N, K, S, sr, part, st);
    return fail(QMV_EINVAL, "internal: no matrix-core kernel for waves=%d ks=%d", p.waves, p.ks);
}

// ---------------------------------------------------------------------------
// Prefill: many activation rows. A workgroup of four waves owns a tile of 64
// activation rows x 256 weight rows and walks K in rounds of one block pair
// (64 columns). Wave w multiplies all four 16-row activation blocks of the
// tile by its own four 16-row weight blocks (rows 64w .. 64w+63 of the tile):
// 4 x 4 MFMA tiles, the block scale applied per block in fp32 as in k_mq.
//   Weights go from global memory to registers and never through LDS: lane
// (G, j) of wave w loads the round's pair of tile row 64w + 16G + j, which
// holds all four k slices of that row; a 4 x 4 transpose across the wave's
// lane rows (xpose4) turns that into slice G of rows 16c + j, c = 0..3, the B
// operands of the wave's four weight blocks, decoded in registers. Each weight
// is decoded once per 64 activation rows.
//   Activations are shared by the four waves through LDS: each round the
// workgroup converts the 64 x 64 activations of the round after next into
// bf16 hi/lo A operands (two records per thread) in one of four LDS buffers,
// with one barrier per two rounds. Loads run two rounds ahead (weights) and
// four rounds ahead (activations) of their use, in two register sets each,
// past the end clamped to the last round (not used).
//   Tiles are numbered with the activation block fastest and each XCD
// (workgroups b with the same b % 8) takes a contiguous share of them: the
// workgroups of one XCD run one range of weight rows against all activation
// blocks side by side, so each weight tile comes into that XCD's L2 once and
// the activations (a few MB) are re-read from L2, not from memory.
//   The products take about 350 vector instructions per wave and round
// against 64 MFMAs, and the two share the SIMD's issue port (an MFMA issues in
// 4 cycles, then runs 16 in the matrix pipe); the scaling FMAs are
// interleaved with the MFMAs, and the block scales are converted to fp32 once
// per round (FMAs that read them as halves issue at a lower rate).
// Requirements (checked by the caller): K % 64 == 0, K > 0, W and ldw 4-byte
// aligned, ldw < 2^32, X 16-byte aligned and ldx % 4 == 0.
// ---------------------------------------------------------------------------
constexpr int GM_MBK = 4;                                  // 16-row activation blocks per tile
constexpr int GM_BM = 16 * GM_MBK, GM_BN = 256, GM_NT = 256;
constexpr int GM_REC = GM_MBK * 2 * 64 / GM_NT;            // A records per thread per round
constexpr int GM_BUF = GM_MBK * 2 * 2 * 1024;              // one round: [m block][block][hi, lo][lane] x 16 B
constexpr int GM_LDS = 4 * GM_BUF;

// WPE: waves per SIMD the register budget is cut for.
template <int QT, int WPE>
__global__ __launch_bounds__(GM_NT) __attribute__((amdgpu_waves_per_eu(WPE))) void k_gemm(
    const uint8_t* __restrict__ W, size_t ldw, const float* __restrict__ X, size_t ldx, float* __restrict__ Y,
    size_t ldy, int M, int N, int K, int tiles_n, int tiles, int per_xcd) {
    using F = MqFmt<QT>;
    constexpr int DW = F::DW, PB = 4 * DW;
    extern __shared__ __align__(16) uint8_t smem[];

    const int t = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (t >= tiles) return;  // uniform over the workgroup
    const int tiles_m = tiles / tiles_n;
    const int m0 = (t % tiles_m) * GM_BM, n0 = (t / tiles_m) * GM_BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = lane >> 4, j = lane & 15;
    const int R = K >> 6;  // rounds (block pairs)

    // ---- weights: this lane's row of the tile (past N: the last row, not stored)
    const int wn = n0 + tid < N ? n0 + tid : N - 1;
    const uint8_t* __restrict__ wrow = W + (uint64_t)(uint32_t)wn * (uint32_t)ldw;
    auto fetch_w = [&](int r, uint32_t (&b)[DW]) __attribute__((always_inline)) {
        load_pair<DW>(wrow + (size_t)(r < R ? r : R - 1) * PB, b);
    };
    // ---- activations: record q = tid + 256 i is slice G = q % 4 of row
    // j = (q % 64) / 4 (operand lane (G, j)), block (q / 64) % 2 and
    // activation block q / 128 of the round. Rows past M are read from row
    // M - 1: a product row depends on its own activation row only, and those
    // rows are not stored.
    const float* xrec[GM_REC];
#pragma unroll
    for (int i = 0; i < GM_REC; ++i) {
        const int q = tid + GM_NT * i;
        // lanes 4r .. 4r+3 of a load take slices 0..3 of one activation row,
        // 64 contiguous bytes (one cache line a lane quad)
        const int rl = q & 63, rb = (q >> 6) & 1, mbk = q >> 7;
        const int m = m0 + mbk * 16 + (rl >> 2);
        xrec[i] = X + (size_t)(m < M ? m : M - 1) * ldx + 32 * rb + F::xoff(rl & 3, 0);
    }
    constexpr int XD = F::xoff(0, 1) - F::xoff(0, 0);  // second 4-float run of a record
    auto fetch_x = [&](int r, f32x4_t (&xr)[GM_REC][2]) __attribute__((always_inline)) {
        const int rr = r < R ? r : R - 1;
#pragma unroll
        for (int i = 0; i < GM_REC; ++i) {
            const float* p = xrec[i] + 64 * rr;
            xr[i][0] = *reinterpret_cast<const f32x4_t*>(p);
            xr[i][1] = *reinterpret_cast<const f32x4_t*>(p + XD);
        }
    };
    auto put_x = [&](int buf, const f32x4_t (&xr)[GM_REC][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < GM_REC; ++i) {
            const int q = tid + GM_NT * i;
            const float v[8] = {xr[i][0][0], xr[i][0][1], xr[i][0][2], xr[i][0][3],
                                xr[i][1][0], xr[i][1][1], xr[i][1][2], xr[i][1][3]};
            uint32_t hw[4], lw[4];
            split_bf16_trunc(v, hw, lw);
            const u32x4 hi = (u32x4){hw[0], hw[1], hw[2], hw[3]};
            const u32x4 lo = (u32x4){lw[0], lw[1], lw[2], lw[3]};
            // its operand slot (G, j) = (slice, row) of the MFMA, at
            // G * 256 + ((j + 4G) % 16) * 16 in its 1 KB (the layout of k_mq)
            const int sg = q & 3, sj = (q & 63) >> 2;
            uint8_t* rec = smem + buf * GM_BUF + (q >> 6) * 2048 + sg * 256 + ((sj + 4 * sg) & 15) * 16;
            *reinterpret_cast<u32x4*>(rec) = hi;
            *reinterpret_cast<u32x4*>(rec + 1024) = lo;
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    // ---- one round: the pair in b (this lane's row) times the A operands in LDS buffer buf
    auto compute = [&](int buf, const uint32_t (&b)[DW]) __attribute__((always_inline)) {
        // both block scales of a row in one dword; dd[c] = those of row 16c + j
        uint32_t dd[4];
        const uint32_t dpk = (b[0] & 0xFFFFu) | (b[QT == QMV_Q4_0 ? 4 : 8] & 0xFFFF0000u);
#pragma unroll
        for (int c = 0; c < 4; ++c) dd[c] = dpk;
        xpose4(dd);
        // v0[c] / v1[c]: code dword(s) of slice G of block 0 / 1 of row 16c + j
        uint32_t v0[4], v1[4], w0[4], w1[4];
        if constexpr (QT == QMV_Q4_0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v0[u] = __builtin_amdgcn_alignbyte(b[u + 1], b[u], 2);
                v1[u] = b[5 + u];
            }
            xpose4(v0);
            xpose4(v1);
        } else {
            // block 0 codes at bytes 2..33 (dwords 0..8, shifted by 2), block 1 at 36..67 (dwords 9..16)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v0[u] = __builtin_amdgcn_alignbyte(b[2 * u + 1], b[2 * u], 2);
                w0[u] = __builtin_amdgcn_alignbyte(b[2 * u + 2], b[2 * u + 1], 2);
                v1[u] = b[9 + 2 * u];
                w1[u] = b[10 + 2 * u];
            }
            xpose4(v0);
            xpose4(w0);
            xpose4(v1);
            xpose4(w1);
        }
        const uint8_t* xa = smem + buf * GM_BUF + G * 256 + ((j + 4 * G) & 15) * 16;
        // eight steps s = (block, activation block) = (s / 4, s % 4): step s
        // reads the A operands of step s + 1, issues its eight MFMAs (four
        // independent hi-then-lo chains) and scales the products of step s - 1
        // into the accumulators; scheduling barriers keep the steps in this
        // order, so that at most two steps' products are live
        bf16x8_t bq[4], ah[2], al[2];
        f32x4_t cc[2][4];
        auto read_a = [&](int s) __attribute__((always_inline)) {
            const uint8_t* ra = xa + (((s & 3) * 2 + (s >> 2)) * 2) * 1024;
            ah[s & 1] = *reinterpret_cast<const bf16x8_t*>(ra);
            al[s & 1] = *reinterpret_cast<const bf16x8_t*>(ra + 1024);
        };
        auto decode = [&](int blk) __attribute__((always_inline)) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if constexpr (QT == QMV_Q4_0)
                    bq[c] = dec_q4(blk ? v1[c] : v0[c]);
                else
                    bq[c] = blk ? dec_q8(v1[c], w1[c]) : dec_q8(v0[c], w0[c]);
            }
        };
        // the block scales as fp32 once per round (the mixed-precision FMA
        // that would read them as halves issues at a lower rate)
        float scf[2][4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            scf[0][c] = half_lo(dd[c]);
            scf[1][c] = half_hi(dd[c]);
            asm volatile("" : "+v"(scf[0][c]), "+v"(scf[1][c]));
        }
        auto scale = [&](int s) __attribute__((always_inline)) {
            const int a = s & 3, blk = s >> 2;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float sc = scf[blk][c];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[a][c][i] = fmaf(sc, cc[s & 1][c][i], acc[a][c][i]);
            }
        };
        decode(0);
        read_a(0);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if (s == 4) {
                // the second block's codes are decoded here, not hoisted above
                pin_regs<4>(v1);
                if constexpr (QT == QMV_Q8_0) pin_regs<4>(w1);
                decode(1);
            }
            if (s + 1 < 8) read_a(s + 1);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                cc[s & 1][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[s & 1], bq[c], (f32x4_t){0.f, 0.f, 0.f, 0.f},
                                                                        0, 0, 0);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                cc[s & 1][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[s & 1], bq[c], cc[s & 1][c], 0, 0, 0);
            if (s > 0) {
                scale(s - 1);
                // the scaling happens here, not sunk below later steps
#pragma unroll
                for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(acc[(s - 1) & 3][c])::"memory");
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        scale(7);
    };

    // ---- pipeline over four LDS buffers: round r's A operands are put into
    // buffer r % 4 two rounds before its products, from activations loaded
    // two rounds before that (register set r % 2); round r's weights are
    // loaded two rounds ahead (set r % 2). A barrier after every second round
    // orders each buffer's writes before its reads and its reads before it is
    // written again. In each round the activation loads go out before the
    // weight loads, so that waiting for the oldest activations never waits
    // for weights issued with them.
    uint32_t wA[DW], wB[DW];
    f32x4_t xA[GM_REC][2], xB[GM_REC][2];
    // (the loads outstanding when the loop is entered are those of two
    // earlier rounds in the loop's own order, so the compiler's wait counts
    // at the top of the loop hold for its first iteration too)
    fetch_x(0, xA);
    fetch_x(1, xB);
    put_x(0, xA);
    put_x(1, xB);
    fetch_x(2, xA);
    fetch_w(0, wA);
    fetch_x(3, xB);
    fetch_w(1, wB);
    lds_barrier();
    auto body = [&](int r, uint32_t (&w)[DW], f32x4_t (&xs)[GM_REC][2], bool sync) __attribute__((always_inline)) {
        compute(r & 3, w);
        put_x((r + 2) & 3, xs);
        fetch_x(r + 4, xs);
        fetch_w(r + 2, w);
        if (sync) lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    int r = 0;
    for (; r + 2 <= R; r += 2) {
        body(r, wA, xA, false);
        body(r + 1, wB, xB, true);
    }
    if (r < R) body(r, wA, xA, false);

    // ---- write the 16 x 16 tiles: lane (G, j) holds rows 4G .. 4G+3 of column j
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int n = n0 + 64 * wave + 16 * c + j;
        if (n >= N) continue;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + a * 16 + 4 * G + i;
                if (m < M) Y[(size_t)m * ldy + n] = acc[a][c][i] * F::OUT_SCALE;
            }
        }
    }
}

template <int QT, int WPE = 2>
int launch_gemm_q(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N,
                  int K, hipStream_t st) {
    const long tiles_m = ((long)M + GM_BM - 1) / GM_BM, tiles_n = ((long)N + GM_BN - 1) / GM_BN;
    const long tiles = tiles_m * tiles_n;
    if (tiles > 0x3FFFFFFF) return fail(QMV_EINVAL, "qmv_gemm: M x N too large");
    const long per_xcd = (tiles + 7) / 8;
    hipLaunchKernelGGL((k_gemm<QT, WPE>), dim3((unsigned)(8 * per_xcd)), dim3(GM_NT), GM_LDS, st, W, ldw, X, ldx, Y,
                       ldy, M, N, K, (int)tiles_n, (int)tiles, (int)per_xcd);
    return check_launch("qmv_gemm tiled kernel");
}

// ---------------------------------------------------------------------------
// Expert-indexed product on the matrix cores, for calls with many pairs
// (batched decode, prefill through the experts). Every workgroup groups the
// launch's pairs by expert in LDS (group_by_expert). Work items are (distinct
// expert u, block of up to 16 of its pairs, tile of 64 weight rows), numbered
// expert by expert; persistent workgroups take them in turn. A wave owns the
// tile's 64 rows: lane (G, j) loads the round's pair of row 16G + j (a
// transpose across lane rows gives the B operands of the four 16-row
// blocks, as in k_gemm) and the activation slice G of pair j's row, which is
// already the A operand lane (G, j) of the MFMA needs: the activations go
// from global memory to registers, are split into bf16 hi/lo there and never
// pass through LDS. KS waves share an item by splitting K into KS parts,
// their partial sums added in part order through LDS at the item's end; with
// KS = 1 each wave runs items on its own. So each selected expert is read
// once per 16 of its pairs, decoded once, and multiplied on the matrix
// cores; per weight the vector work is the decode, a share of the split and
// one FMA of the block scale per 16 x 16 products.
// Requirements (checked by the caller): K % 64 == 0, K / 64 a multiple of
// KS and at least 4 KS, W, ldw and estride 4-byte aligned, ldw < 2^32, X
// 16-byte aligned and ldx % 4 == 0, n_pairs <= IDP_MAX_PAIRS, n_experts <=
// IDP_MAX_EXPERTS.
// ---------------------------------------------------------------------------
constexpr int IQ_NT = 256;
// Buffer resource word 3 for raw 32-bit loads on gfx9 parts, and an offset
// past every buffer the kernel is given (X is below 2 GiB there).
constexpr int IQ_RSRC_WORD3 = 0x00020000;
constexpr uint32_t IQ_X_OFF = 0x80000000u;

template <int QT, int KS>
__global__ __launch_bounds__(IQ_NT) __attribute__((amdgpu_waves_per_eu(2))) void k_idq(
    const uint8_t* __restrict__ W, size_t estride, size_t ldw, int n_experts, const float* __restrict__ X,
    size_t ldx, const uint32_t* __restrict__ ids, int n_pairs, int top_k, float* __restrict__ Y, size_t ldy, int N,
    int K, const float* __restrict__ escale, int* __restrict__ err_flag, int x_bytes) {
    using F = MqFmt<QT>;
    constexpr int DW = F::DW, PB = 4 * DW;
    constexpr int SLOTS = 4 / KS;  // items a workgroup runs side by side
    __shared__ int s_map[IDP_MAX_EXPERTS];
    __shared__ int s_uexp[IDP_MAX_PAIRS];
    __shared__ int s_ustart[IDP_MAX_PAIRS + 1];
    __shared__ int s_cnt[IDP_MAX_PAIRS];
    __shared__ int s_plist[IDP_MAX_PAIRS];
    __shared__ int s_istart[IDP_MAX_PAIRS + 1];  // first item of u
    __shared__ int s_U;
    __shared__ __align__(16) float s_part[KS > 1 ? 4 * 1024 : 4];  // a wave's 16 sums per lane

    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index in a scalar register: the item loop below is then
    // uniform per wave (its trip count derives from it), not exec-masked
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = lane >> 4, j = lane & 15;
    const int U = group_by_expert<IQ_NT>(ids, n_pairs, n_experts, s_map, s_uexp, s_ustart, s_cnt, s_plist, &s_U, Y,
                                         ldy, N, err_flag);
    // The workgroups split an expert's pairs into blocks of 16, so every
    // workgroup must list them in the same order: each expert's pairs sorted
    // by index (the atomics filled them in any order) into s_cnt, free now.
    for (int p = tid; p < s_ustart[U]; p += IQ_NT) {
        const int v = s_plist[p];
        const int u = s_map[ids[v]];
        int rank = 0;
        for (int q = s_ustart[u]; q < s_ustart[u + 1]; ++q) rank += s_plist[q] < v;
        s_cnt[s_ustart[u] + rank] = v;
    }
    __syncthreads();
    const int* __restrict__ plist = s_cnt;
    const int tiles = (N + 63) >> 6;
    if (wave == 0) {  // items of u: blocks of 16 pairs x tiles; exclusive scan
        int base = 0;
        for (int u0 = 0; u0 < U; u0 += 64) {
            const int u = u0 + lane;
            const int c = u < U ? ((s_ustart[u + 1] - s_ustart[u] + 15) >> 4) * tiles : 0;
            int incl = c;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o, 64);
                if (lane >= o) incl += t;
            }
            if (u < U) s_istart[u] = base + incl - c;
            base += __shfl(incl, 63, 64);
        }
        if (lane == 0) s_istart[U] = base;
    }
    __syncthreads();
    const int I = s_istart[U];
    const int P = K >> 6;
    const int kq = wave % KS;  // this wave's part of K: pairs [pb, pb + R)
    const int R = P / KS, pb = kq * R;
    constexpr int XD = F::xoff(0, 1) - F::xoff(0, 0);  // second 4-float run of a record
    // activations through a buffer resource over the launch's x_bytes of X
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(X), 0, x_bytes, IQ_RSRC_WORD3);

    // This wave's items: it0, it0 + stride, ... below I. Every wave of a
    // workgroup runs the same items when KS > 1 (one slot), so the barriers
    // of the part sums match.
    const int it0 = blockIdx.x * SLOTS + wave / KS, stride = gridDim.x * SLOTS;
    const int nit = it0 < I ? (I - it0 + stride - 1) / stride : 0;
    if (nit == 0) return;  // uniform over the workgroup when KS > 1 (one slot); no barrier follows
    // an item's addresses and pairs
    struct Item {
        const uint8_t* wrow;  // this lane's weight row (pair 0)
        uint32_t xoff;        // byte offset in X of this lane's activation slice G of pair j's row
        int e, pbeg, cnt, n0;
    };
    auto decode_item = [&](int it) __attribute__((always_inline)) {
        int u = 0;  // last u with s_istart[u] <= it
        for (int span = IDP_MAX_PAIRS / 2; span > 0; span >>= 1)
            if (u + span < U && s_istart[u + span] <= it) u += span;
        const int rem = it - s_istart[u];
        Item t;
        t.n0 = (rem % tiles) * 64;
        t.pbeg = s_ustart[u] + 16 * (rem / tiles);
        t.cnt = s_ustart[u + 1] - t.pbeg < 16 ? s_ustart[u + 1] - t.pbeg : 16;
        t.e = s_uexp[u];
        const int wn = t.n0 + 16 * G + j < N ? t.n0 + 16 * G + j : N - 1;  // past N: the last row, not stored
        t.wrow = W + (size_t)t.e * estride + (uint64_t)(uint32_t)wn * (uint32_t)ldw + (size_t)pb * PB;
        // lanes past cnt get an offset beyond the buffer: their loads return
        // zeros without touching memory (a product row depends on its own
        // activation row only, and those rows are not stored)
        const int pr = plist[t.pbeg + (j < t.cnt ? j : t.cnt - 1)];
        t.xoff = j < t.cnt ? (uint32_t)(((size_t)(pr / top_k) * ldx + 64 * pb + F::xoff(G, 0)) * 4) : IQ_X_OFF;
        return t;
    };
    // The rounds of this wave's items run as one stream of slots g = k * R4
    // + i (item k, slot i < R4 = R rounded up to a multiple of 4; slots i >=
    // R are skipped). Weights go in super-steps of four rounds: at the first
    // slot of super-step t, the lane loads the four pairs of super-step t + 1
    // (its row's pairs in one burst, so each line of the row is requested
    // while the others are in flight, not again rounds later), into the other
    // of two register sets. Activations go per round, two rounds ahead, in
    // two register sets. The loads cross item boundaries, so a new item starts
    // with its loads in flight; past the last item they repeat the last one's
    // addresses and are not used.
    Item cur = decode_item(it0);
    Item nxt = nit > 1 ? decode_item(it0 + stride) : cur;
    const int R4 = (R + 3) & ~3, T4 = R4 >> 2;
    int kcur = 0;  // item of cur
    auto fetch_w = [&](int sg, uint32_t (&wb)[4][DW]) __attribute__((always_inline)) {  // super-step sg
        const int k = sg / T4, t = sg - k * T4;
        const uint8_t* p = k == kcur ? cur.wrow : nxt.wrow;
#pragma unroll
        for (int q = 0; q < 4; ++q) load_pair<DW>(p + (size_t)(4 * t + q < R ? 4 * t + q : R - 1) * PB, wb[q]);
    };
    auto fetch_x = [&](int g, f32x4_t (&xb)[2][2]) __attribute__((always_inline)) {  // slot g
        const int k = g / R4, r = g - k * R4;
        const uint32_t o = (k == kcur ? cur.xoff : nxt.xoff) + 256u * (uint32_t)(r < R ? r : R - 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            xb[h][0] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, (int)(o + 128 * h), 0, 0));
            xb[h][1] = __builtin_bit_cast(f32x4_t,
                                          __builtin_amdgcn_raw_buffer_load_b128(xrsrc, (int)(o + 128 * h + 4 * XD), 0, 0));
        }
    };
    f32x4_t acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const uint32_t (&b)[DW], const f32x4_t (&xb)[2][2]) __attribute__((always_inline)) {
        // dd[c]: both block scales of row 16c + j; v0/v1 (w0/w1): slice G of its blocks
        uint32_t dd[4];
        const uint32_t dpk = (b[0] & 0xFFFFu) | (b[QT == QMV_Q4_0 ? 4 : 8] & 0xFFFF0000u);
#pragma unroll
        for (int c = 0; c < 4; ++c) dd[c] = dpk;
        xpose4(dd);
        // the block scales as fp32, once (FMAs reading halves issue slower)
        float scf[2][4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            scf[0][c] = half_lo(dd[c]);
            scf[1][c] = half_hi(dd[c]);
            asm volatile("" : "+v"(scf[0][c]), "+v"(scf[1][c]));
        }
        uint32_t v0[4], v1[4], w0[4], w1[4];
        if constexpr (QT == QMV_Q4_0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v0[q] = __builtin_amdgcn_alignbyte(b[q + 1], b[q], 2);
                v1[q] = b[5 + q];
            }
            xpose4(v0);
            xpose4(v1);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v0[q] = __builtin_amdgcn_alignbyte(b[2 * q + 1], b[2 * q], 2);
                w0[q] = __builtin_amdgcn_alignbyte(b[2 * q + 2], b[2 * q + 1], 2);
                v1[q] = b[9 + 2 * q];
                w1[q] = b[10 + 2 * q];
            }
            xpose4(v0);
            xpose4(w0);
            xpose4(v1);
            xpose4(w1);
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const float v[8] = {xb[blk][0][0], xb[blk][0][1], xb[blk][0][2], xb[blk][0][3],
                                xb[blk][1][0], xb[blk][1][1], xb[blk][1][2], xb[blk][1][3]};
            uint32_t hw[4], lw[4];
            split_bf16_trunc(v, hw, lw);
            typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
            const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, (u32x4v){hw[0], hw[1], hw[2], hw[3]});
            const bf16x8_t al = __builtin_bit_cast(bf16x8_t, (u32x4v){lw[0], lw[1], lw[2], lw[3]});
            bf16x8_t bq[4];
            f32x4_t cc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if constexpr (QT == QMV_Q4_0)
                    bq[c] = dec_q4(blk ? v1[c] : v0[c]);
                else
                    bq[c] = blk ? dec_q8(v1[c], w1[c]) : dec_q8(v0[c], w0[c]);
                cc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bq[c], (f32x4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) cc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bq[c], cc[c], 0, 0, 0);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[c][i] = fmaf(scf[blk][c], cc[c][i], acc[c][i]);
            }
        }
    };
    // the item's outputs: lane (G, j) holds rows 4G .. 4G+3 (pairs) of column j
    auto finish = [&]() __attribute__((always_inline)) {
        // (the expert is uniform over the wave: a scalar load, which the
        // vector-load counter that orders the prefetched loads does not see)
        const float sc = (escale ? escale[__builtin_amdgcn_readfirstlane(cur.e)] : 1.f) * F::OUT_SCALE;
        if constexpr (KS > 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) s_part[wave * 1024 + (c * 4 + i) * 64 + lane] = acc[c][i];
            lds_barrier();  // (not __syncthreads: that would also wait for the loads in flight)
            if (kq == 0) {
#pragma unroll
                for (int q = 1; q < KS; ++q)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[c][i] += s_part[(wave + q) * 1024 + (c * 4 + i) * 64 + lane];
            }
        }
        if (kq == 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int n = cur.n0 + 16 * c + j;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 4 * G + i;
                    if (m < cur.cnt && n < N) Y[(size_t)plist[cur.pbeg + m] * ldy + n] = acc[c][i] * sc;
                }
            }
        }
        if constexpr (KS > 1) lds_barrier();  // the part sums are read before the next item writes them
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        ++kcur;
        cur = nxt;
        if (kcur + 1 < nit) nxt = decode_item(it0 + (kcur + 1) * stride);
    };
    uint32_t wA[4][DW], wB[4][DW];
    f32x4_t x0s[2][2], x1s[2][2];
    fetch_w(0, wA);
    fetch_x(0, x0s);
    fetch_x(1, x1s);
    constexpr int XL = 4, WL = 4 * pair_loads<DW>();
    // super-step sg: its four slots with weight set w, the next super-step's
    // weights into set wn; each slot waits for its activations (loads issued
    // after them: the next slot's activations, and the next weights when
    // those went out in between)
    auto superstep = [&](int sg, uint32_t (&w)[4][DW], uint32_t (&wn)[4][DW]) __attribute__((always_inline)) {
        const int t = sg - kcur * T4;  // super-step within the item (past the last item: t >= T4)
        unroll<0, 4>([&](auto Q) {
            constexpr int q = Q;
            if constexpr (q == 0) fetch_w(sg + 1, wn);
            if constexpr (q < 2)
                wait_vmcnt<XL + WL>();
            else
                wait_vmcnt<XL>();
            __builtin_amdgcn_sched_barrier(0);
            const int g = sg * 4 + q;
            if (4 * t + q < R && kcur < nit) compute(w[q], (q & 1) ? x1s : x0s);
            fetch_x(g + 2, (q & 1) ? x1s : x0s);
        });
        if (t == T4 - 1 && kcur < nit) finish();
    };
    const int NS = nit * T4;
    for (int sg = 0; sg < NS; sg += 2) {
        superstep(sg, wA, wB);
        superstep(sg + 1, wB, wA);
    }
}

template <int QT, int KS>
int launch_idq_t(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
                 int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err,
                 hipStream_t st) {
    // items: at most (distinct experts + n_pairs / 16) x 64-row tiles
    const long umax = n_pairs < E ? n_pairs : E;
    const long items = (umax + n_pairs / 16 + 1) * ((N + 63) / 64);
    long grid = (long)num_cus() * 2;  // (three per CU measured slower)
    const long need = (items + 4 / KS - 1) / (4 / KS);
    grid = grid < need ? grid : need;
    grid = grid < 1 ? 1 : grid;
    // the launch's activation rows, in bytes (below 2 GiB: checked by the caller)
    const long x_bytes = (long)(((size_t)(n_pairs / top_k - 1) * ldx + (size_t)K) * 4);
    hipLaunchKernelGGL((k_idq<QT, KS>), dim3((unsigned)grid), dim3(IQ_NT), 0, st, W, es, ldw, E, X, ldx, ids, n_pairs,
                       top_k, Y, ldy, N, K, sc, err, (int)x_bytes);
    return check_launch("qmv_id matrix-core kernel");
}

}  // namespace

// (the workspace size does not depend on the format)
size_t mq_ws_bytes(int M, int N, int K) {
    return M >= 2 && N > 0 && K > 0 ? plan_mq(QMV_Q4_0, M, N, K, SIZE_MAX).ws_bytes : 0;
}

int launch_gemm(int qtype, const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M,
                int N, int K, hipStream_t st) {
    return qtype == QMV_Q4_0 ? launch_gemm_q<QMV_Q4_0>(W, ldw, X, ldx, Y, ldy, M, N, K, st)
                             : launch_gemm_q<QMV_Q8_0>(W, ldw, X, ldx, Y, ldy, M, N, K, st);
}

int launch_idq(int qtype, const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx,
               const uint32_t* ids, int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc,
               int* err, hipStream_t st) {
    const int P = K / 64;
    if (P < 4) return fail(QMV_EINVAL, "internal: K=%d too small for the matrix-core id kernel", K);
    const bool ks4 = P >= 16 && P % 4 == 0;
    if (qtype == QMV_Q4_0)
        return ks4 ? launch_idq_t<QMV_Q4_0, 4>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, st)
                   : launch_idq_t<QMV_Q4_0, 1>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, st);
    return ks4 ? launch_idq_t<QMV_Q8_0, 4>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, st)
               : launch_idq_t<QMV_Q8_0, 1>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, st);
}

int launch_mq(int qtype, const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N,
              int K, void* ws, size_t ws_bytes, hipStream_t st) {
    const MqPlan p = plan_mq(qtype, M, N, K, ws ? ws_bytes : 0);
    return qtype == QMV_Q4_0 ? launch_mq_q<QMV_Q4_0>(W, ldw, X, ldx, Y, ldy, M, N, K, p, (float*)ws, st)
                             : launch_mq_q<QMV_Q8_0>(W, ldw, X, ldx, Y, ldy, M, N, K, p, (float*)ws, st);
}

}  // namespace qmvi
