// qmv.hip — block-quantized weight mat-vec for MI355X (gfx950 / CDNA4).
//
// Implements the C ABI declared in include/qmv.h: the dense products
// qmv_q4_0 / qmv_q8_0 (the `dispatch_qmatmul` calls of the hf2q pages,
// src/inference/models/gemma4/gpu_full_attn.rs, `encode_one_layer`) and the
// expert-indexed product qmv_id (the `quantized_matmul_id_ggml` calls there,
// MoE blocks B11 and B13, over the stacked expert weights of `MlxMoeWeights`
// in src/inference/models/gemma4/model.rs).
//
// Kernels
//   * k_m1_<qtype>   — M = 1 mat-vec, the decode case. Bandwidth-bound: every
//     weight byte is read from HBM once. Each lane streams whole pairs of
//     blocks (36 B for Q4_0, 68 B for Q8_0; 4-byte aligned when rows are) with
//     dwordx4 loads, LPR lanes cover one row, a wave covers 64/LPR rows at a
//     time (RPT rows per lane for ILP and x reuse). The activation vector is
//     staged once per workgroup into LDS (pairs padded to 68 floats so the LPR
//     distinct lanes of a read hit distinct banks). Q4_0 codes are decoded with
//     v_cvt_off_f32_i4 on (byte ^ 0x88): it yields (code - 8) / 16 exactly,
//     so no -8 fold (and no cancellation) is needed; the 1/16 is undone once
//     per output. Each row's partial sums are reduced across its LPR lanes by
//     lane shuffles.
//   * k_generic      — any qtype, 1..16 rows of X, any 2-byte alignment and
//     any K: one wave per weight row, one block per lane per step, 2-byte
//     loads. The fallback for shapes the fast kernels do not take.
//   * k_id           — expert-indexed product. One workgroup per (row tile,
//     (token, slot) pair). The workgroup of the first pair that selects an
//     expert ("leader") gathers every pair selecting the same expert and
//     streams that expert's rows once for all of them; other workgroups exit.
//
// All accumulation is fp32 with a fixed order (no atomics), so outputs are
// bitwise reproducible run to run.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qmv.h"

namespace {

// ---------------------------------------------------------------------------
// Error reporting
// ---------------------------------------------------------------------------
thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QMV_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return QMV_OK;
}

constexpr int QK = 32;

__host__ __device__ constexpr int block_bytes(int qtype) { return qtype == QMV_Q4_0 ? 18 : 34; }

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));

__device__ __forceinline__ float half_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// (code - 8) / 16 for the low nibble of byte B of w, where w already holds
// the code bytes XORed with 0x88 (v_cvt_off_f32_i4 reads bits [3:0] as a
// signed 4-bit value and divides by 16; code ^ 8 sign-extends to code - 8).
template <int B>
__device__ __forceinline__ float nib(uint32_t w) {
    float r;
    if constexpr (B == 0) {
        r = __builtin_amdgcn_cvt_off_f32_i4((int)w);
    } else if constexpr (B == 1) {
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w));
    } else if constexpr (B == 2) {
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w));
    } else {
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w));
    }
    return r;
}

// Signed int8 code in byte B of w, as float.
template <int B>
__device__ __forceinline__ float sbyte(uint32_t w) {
    return (float)(int8_t)(w >> (8 * B));
}

// Compile-time unrolled loop helper.
template <int I, int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        unroll<I + 1, N>(f);
    }
}

// Sum over one Q4_0 block whose 16 code bytes start at byte QB of the
// register window u[] (u = raw ^ 0x88888888, u4 = u >> 4); xv = the block's
// 32 activations. Returns sum_j (code_j - 8) / 16 * x_j.
template <int QB>
__device__ __forceinline__ float q4_block(const uint32_t* u, const uint32_t* u4, const float4* xv) {
    float lo = 0.f, hi = 0.f;
    unroll<0, 4>([&](auto Q) {
        const float4 xl = xv[Q], xh = xv[4 + Q];
        const float xlv[4] = {xl.x, xl.y, xl.z, xl.w}, xhv[4] = {xh.x, xh.y, xh.z, xh.w};
        unroll<0, 4>([&](auto I) {
            constexpr int t = QB + 4 * Q + I;
            lo = fmaf(nib<t % 4>(u[t / 4]), xlv[I], lo);
            hi = fmaf(nib<t % 4>(u4[t / 4]), xhv[I], hi);
        });
    });
    return lo + hi;
}

// Sum over one Q8_0 block whose 32 code bytes start at byte QB of w[].
template <int QB>
__device__ __forceinline__ float q8_block(const uint32_t* w, const float4* xv) {
    float a = 0.f, b = 0.f;
    unroll<0, 8>([&](auto Q) {
        const float4 x4 = xv[Q];
        const float xq[4] = {x4.x, x4.y, x4.z, x4.w};
        unroll<0, 4>([&](auto I) {
            constexpr int t = QB + 4 * Q + I;
            if constexpr (I % 2 == 0)
                a = fmaf(sbyte<t % 4>(w[t / 4]), xq[I], a);
            else
                b = fmaf(sbyte<t % 4>(w[t / 4]), xq[I], b);
        });
    });
    return a + b;
}

// Pair of Q4_0 blocks (36 bytes = 9 dwords). Returns sum over both blocks of
// d_b * sum_j (code - 8)/16 * x_j; the caller multiplies the total by 16.
__device__ __forceinline__ float q4_pair(const uint32_t* r, const float4* xv) {
    uint32_t u[9], u4[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) {
        u[i] = r[i] ^ 0x88888888u;
        u4[i] = u[i] >> 4;
    }
    const float d0 = half_lo(r[0]);
    const float d1 = half_hi(r[4]);
    const float s0 = q4_block<2>(u, u4, xv);        // bytes 2..17
    const float s1 = q4_block<20>(u, u4, xv + 8);  // bytes 20..35
    return fmaf(d1, s1, d0 * s0);
}

// Pair of Q8_0 blocks (68 bytes = 17 dwords).
__device__ __forceinline__ float q8_pair(const uint32_t* r, const float4* xv) {
    const float d0 = half_lo(r[0]);
    const float d1 = half_hi(r[8]);
    const float s0 = q8_block<2>(r, xv);         // bytes 2..33
    const float s1 = q8_block<36>(r, xv + 8);   // bytes 36..67
    return fmaf(d1, s1, d0 * s0);
}

template <int QT>
struct PairTraits;
template <>
struct PairTraits<QMV_Q4_0> {
    static constexpr int DW = 9;  // dwords per pair
    static constexpr float OUT_SCALE = 16.f;
    __device__ static float dot(const uint32_t* r, const float4* xv) { return q4_pair(r, xv); }
};
template <>
struct PairTraits<QMV_Q8_0> {
    static constexpr int DW = 17;
    static constexpr float OUT_SCALE = 1.f;
    __device__ static float dot(const uint32_t* r, const float4* xv) { return q8_pair(r, xv); }
};

template <int DW>
__device__ __forceinline__ void load_pair(const uint8_t* p, uint32_t* r) {
    const u32x4* v = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < DW / 4; ++i) {
#ifdef QMV_LOAD_NT
        u32x4 t = __builtin_nontemporal_load(v + i);
#else
        u32x4 t = v[i];
#endif
        r[4 * i + 0] = t.x;
        r[4 * i + 1] = t.y;
        r[4 * i + 2] = t.z;
        r[4 * i + 3] = t.w;
    }
    if constexpr (DW % 4) {
        r[DW - 1] = reinterpret_cast<const uint32_t*>(p)[DW - 1];
    }
}

// LDS layout of the staged activation row: 64 floats per pair of blocks,
// padded to 68 so that lanes reading different pairs use different banks.
constexpr int XS_PAIR = 68;
constexpr int KMAX_STAGE = 15360;  // largest K staged into LDS by the M = 1 kernels

__host__ __device__ constexpr size_t xs_bytes(int K) { return (size_t)(K / 64) * XS_PAIR * sizeof(float); }

// NT threads copy x (K % 4 == 0, K <= 4 * NT * XCH) into the padded layout:
// every thread first issues all of its 16-byte loads, then stores them, so
// the copy costs one memory latency instead of one per element.
template <int NT, int XCH>
__device__ __forceinline__ void stage_x(float* xs, const float* __restrict__ x, int K) {
    typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
    const int nch = K >> 2;
    f32x4u v[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int c = threadIdx.x + i * NT;
        if (c < nch) v[i] = *reinterpret_cast<const f32x4u*>(x + 4 * c);
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int c = threadIdx.x + i * NT;
        if (c < nch)
            *reinterpret_cast<float4*>(xs + (c >> 4) * XS_PAIR + 4 * (c & 15)) = make_float4(v[i].x, v[i].y, v[i].z, v[i].w);
    }
}

// v + (v of another lane chosen by a DPP control); lanes outside row_mask
// add 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true);
    return v + __builtin_bit_cast(float, t);
}

// Sum of v over aligned groups of LPR lanes, with DPP lane moves only (no
// LDS traffic). The full sum is valid in the last lane of each group
// (lane % LPR == LPR - 1); other lanes hold partial sums.
template <int LPR>
__device__ __forceinline__ float lane_group_sum(float v) {
    if constexpr (LPR >= 2) v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (LPR >= 4) v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) v = dpp_add<0x141>(v);  // row_half_mirror
    if constexpr (LPR >= 16) v = dpp_add<0x140>(v); // row_mirror
    if constexpr (LPR >= 32) v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    if constexpr (LPR >= 64) v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Streams the rows of one M = 1 product through a workgroup: tiles of
// ROWS = (64/LPR) * RPT * WAVES consecutive rows, tiles first_tile,
// first_tile + tile_stride, ... Within a tile, lane j of a row's LPR-lane
// group takes pairs j, j + LPR, ... of that row; each step is one pair of
// RPT rows, and the loads of the next step are issued before the current one
// is decoded (one step of register prefetch). The activation row x is staged
// into LDS after the first loads are in flight. Each row's sum is reduced over
// its lane group and written to y[row] * out_scale.
template <int QT, int LPR, int RPT, int WAVES>
__device__ __forceinline__ void m1_stream(const uint8_t* __restrict__ W, size_t ldw, const float* __restrict__ x,
                                          float* __restrict__ y, int N, int K, long first_tile, long tile_stride,
                                          float out_scale, float* xs) {
    using T = PairTraits<QT>;
    constexpr int DW = T::DW, PB = DW * 4;
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS = GROUPS * RPT * WAVES;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int P = K >> 6;
    const int IPT = (P + LPR - 1) / LPR;  // steps per tile
    const long ntiles = ((long)N + ROWS - 1) / ROWS;
    const long lrow = (long)(wave * GROUPS + g) * RPT;  // this lane's first row within a tile

    long tile = first_tile;
    if (tile >= ntiles) return;  // uniform over the workgroup
    int it = 0;
    uint32_t nxt[RPT][DW];
    auto issue = [&](long tl, int i) {
        const long row0 = tl * ROWS + lrow;
        int p = j + i * LPR;
        p = p < P ? p : P - 1;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const long rr = row0 + r < N ? row0 + r : N - 1;
            load_pair<DW>(W + rr * ldw + (size_t)p * PB, nxt[r]);
        }
    };
    issue(tile, 0);
    stage_x<WAVES * 64, (KMAX_STAGE / 4 + WAVES * 64 - 1) / (WAVES * 64)>(xs, x, K);
    __syncthreads();
    float tot[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) tot[r] = 0.f;
    while (true) {
        uint32_t cur[RPT][DW];
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int d = 0; d < DW; ++d) cur[r][d] = nxt[r][d];
        const int p = j + it * LPR;
        int it2 = it + 1;
        long tile2 = tile;
        if (it2 == IPT) {
            it2 = 0;
            tile2 += tile_stride;
        }
        const bool more = tile2 < ntiles;
        if (more) issue(tile2, it2);
        if (p < P) {
            const float4* xv = reinterpret_cast<const float4*>(xs + p * XS_PAIR);
#pragma unroll
            for (int r = 0; r < RPT; ++r) tot[r] += T::dot(cur[r], xv);
        }
        if (it == IPT - 1) {
            const long row0 = tile * ROWS + lrow;
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const float sum = lane_group_sum<LPR>(tot[r]);
                if (j == LPR - 1 && row0 + r < N) y[row0 + r] = sum * out_scale;
                tot[r] = 0.f;
            }
        }
        if (!more) break;
        tile = tile2;
        it = it2;
    }
}

// ---------------------------------------------------------------------------
// M = 1 dense kernel (fast path). Requires K % 64 == 0, W and ldw 4-aligned.
// Persistent: the grid is sized to the chip and workgroups loop over tiles.
// ---------------------------------------------------------------------------
template <int QT, int LPR, int RPT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_m1(const uint8_t* __restrict__ W, size_t ldw,
                                                   const float* __restrict__ x, float* __restrict__ y, int N, int K) {
    extern __shared__ __align__(16) float xs[];
    m1_stream<QT, LPR, RPT, WAVES>(W, ldw, x, y, N, K, blockIdx.x, gridDim.x, PairTraits<QT>::OUT_SCALE, xs);
}

// ---------------------------------------------------------------------------
// Batched M = 1 kernel: several independent products y_p = W_p x_p in one
// launch (one problem is the plain call). Each problem gets a share of the
// workgroups in proportion to its weight bytes; within a problem, every wave
// gets an equal contiguous range of row groups (a row group = 64/LPR rows,
// LPR lanes per row), so all waves finish together. A lane walks the pairs
// j, j + LPR, ... of its row; the loads of the next two steps are in flight
// while a step is decoded. The workgroup stages its problem's x into LDS
// after issuing its first loads.
// ---------------------------------------------------------------------------
constexpr int MAXB = 16;  // problems per batched launch

struct M1Prob {
    const uint8_t* W;
    const float* x;
    float* y;
    size_t ldw;
    int N, K, lpr, wg0, nwg;
};
struct M1Batch {
    M1Prob p[MAXB];
    int n;
};

template <int LPR>
__device__ __forceinline__ float group_sum_rt(float v) { return lane_group_sum<LPR>(v); }

__device__ __forceinline__ float group_sum_dyn(float v, int lpr) {
    switch (lpr) {
        case 64: return lane_group_sum<64>(v);
        case 32: return lane_group_sum<32>(v);
        case 16: return lane_group_sum<16>(v);
        case 8: return lane_group_sum<8>(v);
        default: return lane_group_sum<4>(v);
    }
}

template <int QT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_m1b(const M1Batch B) {
    extern __shared__ __align__(16) float xs[];
    int pi = 0;
    while (pi + 1 < B.n && (int)blockIdx.x >= B.p[pi + 1].wg0) ++pi;
    const uint8_t* W = B.p[pi].W;
    const float* x = B.p[pi].x;
    float* y = B.p[pi].y;
    const size_t ldw = B.p[pi].ldw;
    const int N = B.p[pi].N, K = B.p[pi].K;
    const long lw = blockIdx.x - B.p[pi].wg0, nwg = B.p[pi].nwg;
    constexpr float OS = PairTraits<QT>::OUT_SCALE;
    switch (B.p[pi].lpr) {
        case 64: m1_stream<QT, 64, 1, WAVES>(W, ldw, x, y, N, K, lw, nwg, OS, xs); break;
        case 32: m1_stream<QT, 32, 1, WAVES>(W, ldw, x, y, N, K, lw, nwg, OS, xs); break;
        case 16: m1_stream<QT, 16, 1, WAVES>(W, ldw, x, y, N, K, lw, nwg, OS, xs); break;
        case 8: m1_stream<QT, 8, 1, WAVES>(W, ldw, x, y, N, K, lw, nwg, OS, xs); break;
        default: m1_stream<QT, 4, 1, WAVES>(W, ldw, x, y, N, K, lw, nwg, OS, xs); break;
    }
}

// ---------------------------------------------------------------------------
// M = 1 one-shot kernel, batched: every wave issues all of its weight loads
// at once, so the whole product costs about one memory latency plus the
// transfer time, and no weight load waits behind arithmetic or a barrier.
//
// Lanes: LPR lanes per row (G = 64 / LPR rows per row group); lane j of a
// group owns ONE pair of blocks (64 activations) of the row, pair
// sg * seg + j, where sg is the wave's segment of K. Rows with more than 64
// pairs are cut into S segments handled by S waves of the workgroup, whose
// partial sums meet in LDS (added in segment order). A row wave owns at most
// MAXI consecutive row groups; all their pair loads (36 or 68 bytes per lane
// each) are issued before anything waits. The activations are read in this
// order: each thread loads its share of x first, then the weights; x goes
// through LDS (once per workgroup) into each lane's registers (its own 64
// values), and every weight pair is reduced as soon as it lands.
// ---------------------------------------------------------------------------
constexpr int MO_WAVES = 8;
constexpr int MO_XCH = 8;  // float4 chunks of x per thread
constexpr int MO_KMAX = MO_WAVES * 64 * MO_XCH * 4;

struct OsProb {
    const uint8_t* W;
    const float* x;
    float* y;
    size_t ldw;
    int N, K;
    int lpr, S;  // lanes per row; K segments (waves) per row group
    int wg0, nwg;
};
struct OsBatch {
    OsProb p[MAXB];
    int n;
};

template <int QT, int MAXI>
__global__ __launch_bounds__(MO_WAVES * 64) void k_m1o(const OsBatch B) {
    using T = PairTraits<QT>;
    constexpr int DW = T::DW, PB = DW * 4;
    typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
    extern __shared__ __align__(16) float xs[];
    __shared__ float red[MO_WAVES][MAXI];
    int pi = 0;
    while (pi + 1 < B.n && (int)blockIdx.x >= B.p[pi + 1].wg0) ++pi;
    const uint8_t* __restrict__ W = B.p[pi].W;
    const float* __restrict__ x = B.p[pi].x;
    float* __restrict__ y = B.p[pi].y;
    const size_t ldw = B.p[pi].ldw;
    const int N = B.p[pi].N, K = B.p[pi].K, LPR = B.p[pi].lpr, S = B.p[pi].S;
    const int lw = blockIdx.x - B.p[pi].wg0, nwg = B.p[pi].nwg;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sg = wave % S, rw = wave / S, R = MO_WAVES / S;
    const int GR = 64 / LPR, g = lane / LPR, j = lane % LPR;
    const int P = K >> 6;
    const int seg = (P + S - 1) / S;
    const int p = sg * seg + j;
    const bool active = j < seg && p < P;
    const int pc = active ? p : P - 1;
    const long RG = ((long)N + GR - 1) / GR;
    const long TR = (long)nwg * R, gr = (long)lw * R + rw;
    const long rg0 = RG * gr / TR, rg1 = RG * (gr + 1) / TR;
    const int nr = (int)(rg1 - rg0);  // <= MAXI (host plan)

    // 1. this thread's share of x
    // (unconditional, clamped, so the compiler can count them and later
    // wait for x alone while the weight loads stay in flight)
    f32x4u xv[MO_XCH];
    const int nch = K >> 2;
#pragma unroll
    for (int i = 0; i < MO_XCH; ++i) {
        const int c = tid + i * MO_WAVES * 64;
        xv[i] = *reinterpret_cast<const f32x4u*>(x + 4 * (c < nch ? c : nch - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    // 2. every weight pair this lane will use
    // (branch-free: surplus slots reload the wave's last row group)
    uint32_t b[MAXI][DW];
    const int last = nr > 0 ? nr - 1 : 0;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        long row = (rg0 + (i < last ? i : last)) * GR + g;
        row = row < N ? row : N - 1;
        load_pair<DW>(W + row * ldw + (size_t)pc * PB, b[i]);
    }
    // Nothing that needs weight data may be scheduled above the x staging.
    __builtin_amdgcn_sched_barrier(0);
    // 3. x into LDS (pairs padded to XS_PAIR floats), then this lane's pair;
    // surplus chunks rewrite the last chunk's slot with the same values.
#pragma unroll
    for (int i = 0; i < MO_XCH; ++i) {
        int c = tid + i * MO_WAVES * 64;
        c = c < nch ? c : nch - 1;
        const int k = 4 * c;
        *reinterpret_cast<float4*>(xs + (k >> 6) * XS_PAIR + (k & 63)) = make_float4(xv[i].x, xv[i].y, xv[i].z, xv[i].w);
    }
    // LDS-only barrier: __syncthreads() would also wait for every weight load
    // in flight (vmcnt(0)), which is exactly what this kernel avoids.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    float4 xr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) xr[i] = reinterpret_cast<const float4*>(xs + pc * XS_PAIR)[i];
    // 4. reduce each pair as it lands
    float v[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const float d = T::dot(b[i], xr);
        v[i] = group_sum_dyn(active ? d : 0.f, LPR);
    }
    if (S == 1) {
        if (j == LPR - 1) {
#pragma unroll
            for (int i = 0; i < MAXI; ++i) {
                const long row = (rg0 + i) * GR + g;
                if (i < nr && row < N) y[row] = v[i] * T::OUT_SCALE;
            }
        }
        return;
    }
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < MAXI; ++i) red[wave][i] = v[i];
    }
    __syncthreads();
    if (sg == 0 && lane == 63) {
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            float t = v[i];
            for (int s2 = 1; s2 < S; ++s2) t += red[wave + s2][i];
            const long row = rg0 + i;
            if (i < nr && row < N) y[row] = t * T::OUT_SCALE;
        }
    }
}

// ---------------------------------------------------------------------------
// M = 1 x-stationary kernel.
//
// Every lane owns one pair of blocks (64 activations) of K for the whole
// kernel and keeps those activations in registers; weight rows stream past.
// A row's P = K/64 pairs are split into S segments of `seg` pairs; a wave
// covers one segment of 64/LPR rows (LPR lanes per row, lane j of a row
// group holding pair s*seg + j), RPT rows per lane per step. The S waves of
// a segment group hold the same rows; their partial sums meet in LDS. The
// workgroup has S * WR waves (WR row-waves per segment). Loads run two steps
// ahead of the arithmetic.
// ---------------------------------------------------------------------------
struct XsPlan {
    int S, seg, WR;
};

template <int QT, int LPR, int RPT>
__global__ __launch_bounds__(512) void k_m1x(const uint8_t* __restrict__ W, size_t ldw, const float* __restrict__ x,
                                              float* __restrict__ y, int N, int K, XsPlan plan, float out_scale) {
    using T = PairTraits<QT>;
    constexpr int DW = T::DW, PB = DW * 4;
    constexpr int GROUPS = 64 / LPR;
    __shared__ float red[2][8][GROUPS * RPT];  // [step parity][wave][row slot]
    const int S = plan.S, seg = plan.seg, WR = plan.WR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int s = wave % S, rw = wave / S;
    const int g = lane / LPR, j = lane % LPR;
    const int P = K >> 6;
    const int pidx = s * seg + j;
    const bool active = j < seg && pidx < P;
    const int pc = active ? pidx : 0;
    const int ROWS_STEP = WR * GROUPS * RPT;
    const long nsteps = ((long)N + ROWS_STEP - 1) / ROWS_STEP;
    const long lrow = (long)(rw * GROUPS + g) * RPT;

    // This lane's 64 activations, kept in registers.
    float4 xr[16];
    {
        const float4* xp = reinterpret_cast<const float4*>(x + (size_t)pc * 64);
#pragma unroll
        for (int i = 0; i < 16; ++i) xr[i] = active ? xp[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    auto issue = [&](long step, uint32_t (&b)[RPT][DW]) {
        const long row0 = step * ROWS_STEP + lrow;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            long rr = row0 + r;
            rr = rr < N ? rr : N - 1;
            load_pair<DW>(W + rr * ldw + (size_t)pc * PB, b[r]);
        }
    };
    auto finish = [&](long step, const uint32_t (&b)[RPT][DW], int parity) {
        float v[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) v[r] = active ? T::dot(b[r], xr) : 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) v[r] = lane_group_sum<LPR>(v[r]);
        const long row0 = step * ROWS_STEP + lrow;
        if (S == 1) {
            if (j == LPR - 1) {
#pragma unroll
                for (int r = 0; r < RPT; ++r)
                    if (row0 + r < N) y[row0 + r] = v[r] * out_scale;
            }
            return;
        }
        if (j == LPR - 1) {
#pragma unroll
            for (int r = 0; r < RPT; ++r) red[parity][wave][g * RPT + r] = v[r];
        }
        __syncthreads();
        if (s == 0 && j == LPR - 1) {
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                float acc = v[r];
                for (int q = 1; q < S; ++q) acc += red[parity][wave + q][g * RPT + r];
                if (row0 + r < N) y[row0 + r] = acc * out_scale;
            }
        }
    };

    long step = blockIdx.x;
    if (step >= nsteps) return;  // uniform over the workgroup
    const long stride = gridDim.x;
    uint32_t ba[RPT][DW], bb[RPT][DW];
    issue(step, ba);
    if (step + stride < nsteps) issue(step + stride, bb);
    int parity = 0;
    while (true) {
        finish(step, ba, parity);
        parity ^= 1;
        if (step + 2 * stride < nsteps) issue(step + 2 * stride, ba);
        step += stride;
        if (step >= nsteps) break;
        finish(step, bb, parity);
        parity ^= 1;
        if (step + 2 * stride < nsteps) issue(step + 2 * stride, bb);
        step += stride;
        if (step >= nsteps) break;
    }
}

// ---------------------------------------------------------------------------
// M = 1 Q4_0 kernel on the matrix cores (v_mfma_f32_16x16x32_f16).
//
// A wave owns a tile of 16 weight rows (MFMA columns j = lane % 16) and a
// segment of each row's block pairs. Lane group G = lane / 16 streams pair
// q = p0 + 4t + G of row j at step t (36 bytes, two blocks), so the four lane
// groups each feed their own block into one of the four 8-wide k slices of
// every MFMA: slice G of MFMA u carries qs dword u of the lane's block, i.e.
// 8 codes, as exact fp16 values (code - 8). The A operand is block diagonal:
// row 4G + 0 holds the hi fp16 part and row 4G + 1 the lo fp16 part of the
// matching activations in slice G, every other entry is zero. After the four
// MFMAs of a block, lane (G, j) holds that block's sums for row j in D rows
// 4G (hi) and 4G + 1 (lo), so the fp16 block scale is applied in fp32 right
// there: acc += d * (D[4G] + D[4G+1]).
//
// The activations are split once per workgroup (x * 2^s = hi + lo with hi,
// lo fp16 and 2^s bringing max |x| into [2^14, 2^15)) and stored in LDS in
// the order the A operands read them: per block 128 bytes = 4 dwords u x
// {hi, lo} x 8 halves. Products of fp16 values are exact in fp32 and hi + lo
// carries 22 bits of each activation, so the result is fp32-accurate.
// ---------------------------------------------------------------------------
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 8 codes of one qs dword -> fp16 (code - 8), in the element order
// [4u+0, 4u+2, 4u+1, 4u+3, 20+4u-4.., ...] = lo nibbles of bytes 0,2,1,3 then
// hi nibbles of bytes 0,2,1,3 (u = the dword's index within the block).
__device__ __forceinline__ half8_t q4_codes_f16(uint32_t q) {
    const uint32_t M = 0x000F000Fu, MAGIC = 0x64006400u;  // fp16 1024 + nibble
    const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t v0 = __builtin_bit_cast(half2_t, (q & M) | MAGIC) + bias;
    const half2_t v1 = __builtin_bit_cast(half2_t, ((q >> 8) & M) | MAGIC) + bias;
    const half2_t v2 = __builtin_bit_cast(half2_t, ((q >> 4) & M) | MAGIC) + bias;
    const half2_t v3 = __builtin_bit_cast(half2_t, ((q >> 12) & M) | MAGIC) + bias;
    half8_t r;
    r[0] = v0[0]; r[1] = v0[1]; r[2] = v1[0]; r[3] = v1[1];
    r[4] = v2[0]; r[5] = v2[1]; r[6] = v3[0]; r[7] = v3[1];
    return r;
}

// Byte offset within a block's 128-byte LDS record of activation e (0..31),
// piece p (0 = hi, 1 = lo); matches q4_codes_f16's element order.
__device__ __forceinline__ int xh_offset(int e, int p) {
    const int hi = e >> 4, kk = e & 15, u = kk >> 2, r = kk & 3;
    const int pos = hi * 4 + ((r & 1) << 1 | (r >> 1));  // 0,2,1,3 -> 0,1,2,3 order
    return u * 32 + p * 16 + pos * 2;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Split x (K floats) into scaled fp16 hi/lo pairs in the MFMA A-operand
// order. Returns the power-of-two exponent s (x was multiplied by 2^s).
// Called by all threads of the workgroup; ends with a barrier.
__device__ int stage_x_f16(uint8_t* xh, const float* __restrict__ x, int K, float* red) {
    float m = 0.f;
    for (int k = threadIdx.x; k < K; k += blockDim.x) m = fmaxf(m, fabsf(x[k]));
    m = wave_max(m);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = red[0];
    for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w]);
    int s = 0;
    if (m > 0.f && m <= 3.4e38f) {
        int e;
        frexpf(m, &e);  // m in [2^(e-1), 2^e)
        s = 15 - e;
        s = s > 126 ? 126 : (s < -126 ? -126 : s);
    }
    for (int k = threadIdx.x; k < K; k += blockDim.x) {
        const float v = ldexpf(x[k], s);
        const _Float16 h = (_Float16)v;
        const _Float16 l = (_Float16)(v - (float)h);
        uint8_t* rec = xh + (size_t)(k >> 5) * 128;
        *reinterpret_cast<_Float16*>(rec + xh_offset(k & 31, 0)) = h;
        *reinterpret_cast<_Float16*>(rec + xh_offset(k & 31, 1)) = l;
    }
    __syncthreads();
    return s;
}

// Plan: tiles of 16 rows; each row's P pairs in S segments of `seg` pairs;
// a workgroup has S * WR waves and works on WR tiles at a time.
struct MhPlan {
    int S, seg, WR;
};

__global__ __launch_bounds__(1024) void k_m1h(const uint8_t* __restrict__ W, size_t ldw, const float* __restrict__ x,
                                              float* __restrict__ y, int N, int K, MhPlan plan, float out_scale) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[2][16][16];  // [tile parity][wave][row]
    const int S = plan.S, seg = plan.seg, WR = plan.WR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sgi = wave % S, rw = wave / S;
    const int G = lane >> 4, j = lane & 15;
    const int P = K >> 6;
    const int p0 = sgi * seg;
    const int p1 = p0 + seg < P ? p0 + seg : P;
    const int nsteps = (seg + 3) >> 2;  // the same for every wave of the grid
    const long ntiles = ((long)N + 15) / 16;
    const long tstride = (long)gridDim.x * WR;
    const long tile0 = (long)blockIdx.x * WR + rw;
    // Every wave walks the same number of (tile, step) items so that the
    // workgroup's barriers line up; items past the last tile are masked.
    const long rounds = (ntiles + tstride - 1) / tstride;
    const long nitems = rounds * nsteps;
    // A-operand lanes: row i = lane % 16 with i / 4 == G and i % 4 < 2.
    const bool a_lane = (j >> 2) == G && (j & 3) < 2;
    const int a_piece = j & 1;

    // Issue cursor (tile, step) runs two items ahead of the compute cursor.
    long itile = tile0;
    int istep = 0;
    long issued = 0;
    auto issue = [&](uint32_t (&b)[9]) {
        if (issued < nitems) {
            long row = itile * 16 + j;
            row = row < N ? row : N - 1;
            int q = p0 + 4 * istep + G;
            q = q < p1 ? q : p1 - 1;
            q = q > 0 ? q : 0;
            load_pair<9>(W + row * ldw + (size_t)q * 36, b);
        }
        ++issued;
        if (++istep == nsteps) {
            istep = 0;
            itile += tstride;
        }
    };

    uint32_t b0[9], b1[9];
    issue(b0);
    issue(b1);
    const int sx = stage_x_f16(smem, x, K, &red[0][0][0]);
    const float yscale = ldexpf(out_scale, -sx);

    half8_t a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = (half8_t){0, 0, 0, 0, 0, 0, 0, 0};
    float acc = 0.f;
    int parity = 0;
    long ptile = tile0;
    int pstep = 0;

    auto process = [&](const uint32_t (&r)[9]) {
        const bool tile_ok = ptile < ntiles;
        const int q = p0 + 4 * pstep + G;
        const bool valid = tile_ok && q < p1;
#pragma unroll
        for (int R = 0; R < 2; ++R) {
            const int bk = 2 * q + R;
            if (a_lane) {
                const uint8_t* rec = smem + (size_t)(valid ? bk : 0) * 128 + a_piece * 16;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const half8_t v = *reinterpret_cast<const half8_t*>(rec + u * 32);
                    a[u] = valid ? v : (half8_t){0, 0, 0, 0, 0, 0, 0, 0};
                }
            }
            uint32_t qd[4];
            float d;
            if (R == 0) {
#pragma unroll
                for (int u = 0; u < 4; ++u) qd[u] = __builtin_amdgcn_alignbyte(r[u + 1], r[u], 2);
                d = half_lo(r[0]);
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) qd[u] = r[5 + u];
                d = half_hi(r[4]);
            }
            f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u)
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[u], q4_codes_f16(qd[u]), c, 0, 0, 0);
            if (valid) acc = fmaf(d, c[0] + c[1], acc);
        }
        if (pstep == nsteps - 1) {
            // Sum the four lane groups (block slices) of each row.
            float v = acc + __shfl_xor(acc, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc = 0.f;
            const long row = ptile * 16 + j;
            if (S == 1) {
                if (tile_ok && G == 0 && row < N) y[row] = v * yscale;
            } else {
                if (G == 0) red[parity][wave][j] = v;
                __syncthreads();
                if (tile_ok && sgi == 0 && G == 0 && row < N) {
                    float tot = v;
                    for (int q2 = 1; q2 < S; ++q2) tot += red[parity][wave + q2][j];
                    y[row] = tot * yscale;
                }
                parity ^= 1;
            }
            pstep = 0;
            ptile += tstride;
        } else {
            ++pstep;
        }
    };

    for (long it = 0; it < nitems; it += 2) {
        process(b0);
        issue(b0);
        if (it + 1 < nitems) {
            process(b1);
            issue(b1);
        }
    }
}

MhPlan make_mh_plan(int N, int K, int ncu, int target_waves_per_cu) {
    const int P = K / 64;
    const long ntiles = ((long)N + 15) / 16;
    // Segments: enough (tile, segment) waves to fill the chip, each at least
    // 4 pairs per lane group step and at most 16 segments.
    long want = (long)ncu * target_waves_per_cu;
    int S = 1;
    while (S < 16 && ntiles * S < want && (P + 2 * S - 1) / (2 * S) >= 4) S *= 2;
    MhPlan pl;
    pl.S = S;
    pl.seg = (P + S - 1) / S;
    pl.WR = S >= 8 ? 1 : 8 / S;
    return pl;
}

// ---------------------------------------------------------------------------
// Q4_0 codes as matrix-core operands. One qs dword holds 8 codes: the low
// nibbles of its bytes are block elements 4u..4u+3, the high nibbles elements
// 16+4u..16+4u+3 (u = the dword's index in the block). q4_dec turns them
// into eight exact fp16 values code - 8 in the order
//   [4u, 4u+2, 4u+1, 4u+3, 16+4u, 16+4u+2, 16+4u+1, 16+4u+3].
// A low nibble n as the low byte of an fp16 whose high byte is 0x64 reads as
// 1024 + n; a high nibble left in bits 4..7 under the high byte 0x54 reads as
// 64 + n. v_perm_b32 builds both pairs of a dword from the masked code bytes
// and a register holding the two high bytes, and one packed fp16 add removes
// the offset exactly: 2 AND, 4 v_perm_b32 and 4 v_pk_add_f16 per dword.
// ---------------------------------------------------------------------------
__device__ __forceinline__ half8_t q4_dec(uint32_t q) {
    const half2_t blo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t bhi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t EXPB = 0x5464u;  // byte 4 of {EXPB, v} = 0x64, byte 5 = 0x54
    const uint32_t lo = q & 0x0F0F0F0Fu, hi = q & 0xF0F0F0F0u;
    const half2_t t0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(EXPB, lo, 0x04020400u)) + blo;
    const half2_t t1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(EXPB, lo, 0x04030401u)) + blo;
    const half2_t t2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(EXPB, hi, 0x05020500u)) + bhi;
    const half2_t t3 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(EXPB, hi, 0x05030501u)) + bhi;
    return (half8_t){t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
}

// ---------------------------------------------------------------------------
// M = 1 Q4_0 on the matrix cores, batched (one launch serves up to 16
// independent products y_p = W_p x_p).
//
// A wave owns a tile of 16 weight rows (MFMA column n = lane % 16) and a
// segment of each row's block pairs; lane group G = lane / 16 streams pair
// p0 + 4t + G of row n at step t (36 bytes). For block R of that pair, MFMA u
// (u = 0..3) takes qs dword u of the lane's block as its B slice G. The A
// operand is block diagonal: row 4G holds the hi and row 4G + 1 the lo fp16
// part of the eight activations that slice G multiplies, every other entry is
// zero, so after the four MFMAs lane (G, n) holds in D rows 4G and 4G + 1 the
// block's dot product for row n, and the block's scale is applied in fp32.
// The multiply-adds run on the matrix cores; the vector ALUs only unpack
// codes (about 1.3 instructions per weight).
//
// Activations: each workgroup converts its problem's x once, in one pass,
// into LDS records laid out as the A operands read them (MQ_PAIR bytes per
// pair of blocks: block R x dword u x {hi, lo} x 8 fp16, then the two blocks'
// factors 2^-s, then padding that staggers consecutive pairs over the LDS
// banks). Block b is scaled by the power of two 2^s that brings its largest
// |x| into [2^14, 2^15) and split as x * 2^s = hi + lo; fp16 products are
// exact in fp32 and hi + lo keeps 22 bits of every activation. One zero
// record after the last pair stands in for pairs past the end of a row.
//
// Work split: a tile's pairs are cut into S segments (S waves per tile,
// T = WAVES / S tiles per workgroup pass); segment partial sums meet in LDS
// and are added in segment order, so results do not depend on timing. The
// grid is persistent: workgroup w of a problem takes tile groups w, w + nwg,
// ... Weight loads run two steps ahead of the arithmetic.
// ---------------------------------------------------------------------------
constexpr int MQ_PAIR = 288;
constexpr int MQ_KMAX = 32768;

__host__ __device__ constexpr size_t mq_lds_bytes(int K) { return (size_t)(K / 64 + 1) * MQ_PAIR; }

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
    return fmaxf(v, __builtin_bit_cast(float, t));
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Converts x[0..K) (K % 64 == 0) into the A-operand records at xs. Four
// consecutive threads share a block: thread u of it holds the activations of
// qs dword u (elements 4u..4u+3 and 16+4u..16+4u+3). Ends without a barrier.
__device__ __forceinline__ void stage_xq(uint8_t* xs, const float* __restrict__ x, int K) {
    typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
    const int nb = K >> 5;
    for (int i = threadIdx.x; i < nb * 4; i += blockDim.x) {
        const int b = i >> 2, u = i & 3;
        const f32x4u l4 = *reinterpret_cast<const f32x4u*>(x + (size_t)b * 32 + 4 * u);
        const f32x4u h4 = *reinterpret_cast<const f32x4u*>(x + (size_t)b * 32 + 16 + 4 * u);
        const float v[8] = {l4.x, l4.z, l4.y, l4.w, h4.x, h4.z, h4.y, h4.w};
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
        m = dpp_max<0xB1>(m);  // quad_perm [1,0,3,2]
        m = dpp_max<0x4E>(m);  // quad_perm [2,3,0,1]
        int s = 0;
        if (m > 0.f && m <= 3.4e38f) {
            int ex;
            frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
            s = 15 - ex;
            s = s > 126 ? 126 : (s < -126 ? -126 : s);
        }
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            _Float16 h[2], l[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float a = ldexpf(v[2 * k + c], s);
                h[c] = (_Float16)a;
                float r = a - (float)h[c];
                r = r == r ? r : 0.f;  // hi = +-inf or nan carries the value alone
                l[c] = (_Float16)r;
            }
            hw[k] = pack_h2(h[0], h[1]);
            lw[k] = pack_h2(l[0], l[1]);
        }
        uint8_t* rec = xs + (size_t)(b >> 1) * MQ_PAIR + (b & 1) * 128 + u * 32;
        *reinterpret_cast<u32x4*>(rec) = (u32x4){hw[0], hw[1], hw[2], hw[3]};
        *reinterpret_cast<u32x4*>(rec + 16) = (u32x4){lw[0], lw[1], lw[2], lw[3]};
        if (u == 0) *reinterpret_cast<float*>(xs + (size_t)(b >> 1) * MQ_PAIR + 256 + (b & 1) * 4) = ldexpf(1.f, -s);
    }
    uint8_t* zr = xs + (size_t)(K >> 6) * MQ_PAIR;
    for (int i = threadIdx.x; i < MQ_PAIR / 16; i += blockDim.x)
        *reinterpret_cast<u32x4*>(zr + 16 * i) = (u32x4){0u, 0u, 0u, 0u};
}

struct MqProb {
    const uint8_t* W;
    const float* x;
    float* y;
    size_t ldw;
    int N, K;
    int S;     // segments per tile (divides WAVES)
    int segP;  // pairs per segment
    int wg0, nwg;
};
struct MqBatch {
    MqProb p[MAXB];
    int n;
};

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_m1q(const MqBatch B) {
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* xs = smem;
    __shared__ float red[2][WAVES][16];
    int pi = 0;
    while (pi + 1 < B.n && (int)blockIdx.x >= B.p[pi + 1].wg0) ++pi;
    const uint8_t* __restrict__ W = B.p[pi].W;
    const float* __restrict__ x = B.p[pi].x;
    float* __restrict__ y = B.p[pi].y;
    const size_t ldw = B.p[pi].ldw;
    const int N = B.p[pi].N, K = B.p[pi].K, S = B.p[pi].S, segP = B.p[pi].segP;
    const int lw = blockIdx.x - B.p[pi].wg0, nwg = B.p[pi].nwg;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = lane >> 4, n = lane & 15;
    const int T = WAVES / S;
    const int ts = wave / S, sg = wave % S;
    const int P = K >> 6;
    const int p0 = sg * segP;
    const int nsteps = (segP + 3) >> 2;
    const long ntiles = ((long)N + 15) / 16;
    const long ntg = (ntiles + T - 1) / T;
    const long nk = lw < ntg ? (ntg - lw + nwg - 1) / nwg : 0;
    const long nitems = nk * nsteps;  // the same for every wave of the workgroup
    const bool a_lane = (n >> 2) == G && (n & 3) < 2;
    const int a_off = (n & 1) * 16;  // hi or lo piece

    long ik = 0;
    int ist = 0;
    long issued = 0;
    auto issue = [&](uint32_t (&b)[9]) {
        if (issued < nitems) {
            const long tile = (lw + ik * nwg) * T + ts;
            long row = tile * 16 + n;
            row = row < N ? row : N - 1;
            int p = p0 + 4 * ist + G;
            p = p < P ? p : P - 1;
            load_pair<9>(W + row * ldw + (size_t)p * 36, b);
        }
        ++issued;
        if (++ist == nsteps) {
            ist = 0;
            ++ik;
        }
    };
    uint32_t b0[9], b1[9];
    issue(b0);
    issue(b1);
    stage_xq(xs, x, K);
    __syncthreads();

    half8_t a0[4], a1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        a0[u] = (half8_t){0, 0, 0, 0, 0, 0, 0, 0};
        a1[u] = a0[u];
    }
    float acc = 0.f;
    long pk = 0;
    int pst = 0, parity = 0;
    auto process = [&](const uint32_t (&r)[9]) {
        const int q = 4 * pst + G;
        const int p = p0 + q;
        const bool valid = q < segP && p < P;
        const uint8_t* rec = xs + (size_t)(valid ? p : P) * MQ_PAIR;
        if (a_lane) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a0[u] = *reinterpret_cast<const half8_t*>(rec + u * 32 + a_off);
                a1[u] = *reinterpret_cast<const half8_t*>(rec + 128 + u * 32 + a_off);
            }
        }
        const float2 xsc = *reinterpret_cast<const float2*>(rec + 256);
        f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u)
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[u], q4_dec(__builtin_amdgcn_alignbyte(r[u + 1], r[u], 2)),
                                                        c0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1[u], q4_dec(r[5 + u]), c1, 0, 0, 0);
        const float s0 = valid ? half_lo(r[0]) * xsc.x : 0.f;
        const float s1 = valid ? half_hi(r[4]) * xsc.y : 0.f;
        acc = fmaf(s0, c0[0] + c0[1], acc);
        acc = fmaf(s1, c1[0] + c1[1], acc);
        if (++pst == nsteps) {
            float v = acc + __shfl_xor(acc, 16, 64);
            v += __shfl_xor(v, 32, 64);
            acc = 0.f;
            const long tile = (lw + pk * nwg) * T + ts;
            const long row = tile * 16 + n;
            const bool ok = tile < ntiles && row < N;
            if (S == 1) {
                if (G == 0 && ok) y[row] = v;
            } else {
                if (G == 0) red[parity][wave][n] = v;
                __syncthreads();
                if (sg == 0 && G == 0 && ok) {
                    float t = v;
                    for (int s2 = 1; s2 < S; ++s2) t += red[parity][wave + s2][n];
                    y[row] = t;
                }
                parity ^= 1;
            }
            pst = 0;
            ++pk;
        }
    };
    for (long it = 0; it < nitems; it += 2) {
        process(b0);
        issue(b0);
        if (it + 1 < nitems) {
            process(b1);
            issue(b1);
        }
    }
}

// ---------------------------------------------------------------------------
// M = 2..16 kernel on the matrix cores (v_mfma_f32_16x16x32_f16).
//
// One MFMA multiplies 16 activation rows (A, padded with zero rows) by one
// block of 16 weight rows (B): lane (G, j) of B supplies qs dword G of the
// block of weight row j as 8 exact fp16 codes (code - 8). Every lane streams
// whole 36-byte block pairs (pair 4t + G of its row at step t), so after the
// loads each of the four lane groups holds different blocks; two 4 x 4
// transposes across the four 16-lane rows (v_permlane16_swap, then
// v_permlane32_swap) hand lane group G dword G of all eight blocks of the
// step, and the same transposes gather the eight block scales. Each block
// takes two MFMAs (x split into fp16 hi + lo), and the fp16 block scale is
// applied in fp32 to the 16 x 16 partial: acc += d[row, block] * D.
//
// Activations are staged per chunk of 512 columns into LDS (double
// buffered), already split into hi/lo and ordered as the A operands read
// them; each activation row of a chunk is scaled by a power of two that puts
// its largest magnitude in [2^14, 2^15) (fp16 range), undone when the chunk's
// partial sums are added to the accumulator.
// ---------------------------------------------------------------------------
constexpr int MM_KC = 512;                        // activation columns per staged chunk
constexpr int MM_CHUNK_BYTES = (MM_KC / 32) * 2 * 1024;  // blocks x {hi, lo} x 16 rows x 4 slices x 16 B

// 4 x 4 transpose across the four 16-lane rows: on entry lane row R holds
// v[c] = element (R, c); on exit it holds v[c] = element (c, R).
__device__ __forceinline__ void xpose4(uint32_t* v) {
    auto a = __builtin_amdgcn_permlane16_swap(v[0], v[1], false, false);
    auto b = __builtin_amdgcn_permlane16_swap(v[2], v[3], false, false);
    auto c = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
    v[0] = c[0];
    v[2] = c[1];
    v[1] = d[0];
    v[3] = d[1];
}

// Position (in halves) of block element e within its 8-half A/B slice.
__device__ __forceinline__ int slice_pos(int e) {
    const int r = e & 3;
    return ((e >> 4) << 2) + ((r & 1) << 1 | (r >> 1));
}

template <int WAVES, int TW>
__global__ __launch_bounds__(WAVES * 64) void k_mm(const uint8_t* __restrict__ W, size_t ldw,
                                                   const float* __restrict__ X, size_t ldx, float* __restrict__ Y,
                                                   size_t ldy, int M, int N, int K) {
    extern __shared__ __align__(16) uint8_t smem[];   // 2 activation chunks
    __shared__ float s_scale[2][16];                 // per chunk buffer: 2^-s for each activation row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = lane >> 4, j = lane & 15;
    const int P = K >> 6;
    const int nchunks = (K + MM_KC - 1) / MM_KC;
    const long row_base = ((long)blockIdx.x * WAVES + wave) * 16 * TW;

    // ---- activation staging: thread t covers 16 columns of one row ----
    auto stage = [&](int c, int buf) {
        uint8_t* dst = smem + buf * MM_CHUNK_BYTES;
        const int t = threadIdx.x;
        for (int base = 0; base < 16 * 32; base += WAVES * 64) {
            const int u = base + t;             // 0..511: row m = u / 32, columns (u % 32) * 16 ..
            const int m = u >> 5, c0 = (u & 31) * 16;
            float v[16];
            float mx = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int k = c * MM_KC + c0 + e;
                v[e] = (m < M && k < K) ? X[(size_t)m * ldx + k] : 0.f;
                mx = fmaxf(mx, fabsf(v[e]));
            }
            // max over the 32 threads of this row (a half wave)
#pragma unroll
            for (int off = 16; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 32));
            int sh = 0;
            if (mx > 0.f && mx <= 3.4e38f) {
                int ex;
                frexpf(mx, &ex);
                sh = 15 - ex;
                sh = sh > 126 ? 126 : (sh < -126 ? -126 : sh);
            }
            if ((u & 31) == 0) s_scale[buf][m] = ldexpf(1.f, -sh);
            const int blk = c0 >> 5, e0 = c0 & 31;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float xv = ldexpf(v[e], sh);
                const _Float16 h = (_Float16)xv;
                const _Float16 l = (_Float16)(xv - (float)h);
                const int el = e0 + e, g = (el & 15) >> 2;
                uint8_t* rec = dst + (size_t)blk * 2048 + m * 64 + g * 16 + slice_pos(el) * 2;
                *reinterpret_cast<_Float16*>(rec) = h;
                *reinterpret_cast<_Float16*>(rec + 1024) = l;
            }
        }
    };

    // ---- weight loads: one pair per lane per tile per step ----
    const int steps_per_chunk = MM_KC / 256;
    const int nsteps = nchunks * steps_per_chunk;
    auto issue = [&](int step, uint32_t (&b)[TW][9]) {
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
            long row = row_base + tw * 16 + j;
            row = row < N ? row : N - 1;
            int q = step * 4 + G;
            q = q < P ? q : P - 1;
            load_pair<9>(W + row * ldw + (size_t)q * 36, b[tw]);
        }
    };

    uint32_t b0[TW][9], b1[TW][9];
    issue(0, b0);
    if (nsteps > 1) issue(1, b1);
    stage(0, 0);
    __syncthreads();

    f32x4_t acc[TW], cacc[TW];
#pragma unroll
    for (int tw = 0; tw < TW; ++tw) {
        acc[tw] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        cacc[tw] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }

    auto compute = [&](int step, uint32_t (&r)[TW][9]) {
        const int c = step / steps_per_chunk, buf = c & 1;
        const uint8_t* xa = smem + buf * MM_CHUNK_BYTES + (step % steps_per_chunk) * 8 * 2048 + j * 64 + G * 16;
        const int q = step * 4 + G;
        const bool valid = q < P;
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
            // qs dwords of this lane's two blocks, then hand out slices
            uint32_t v0[4], v1[4], dd[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v0[u] = __builtin_amdgcn_alignbyte(r[tw][u + 1], r[tw][u], 2);
                v1[u] = r[tw][5 + u];
            }
            // both block scales (fp16) packed in one dword; zero for pairs past K
            const uint32_t dpk = valid ? ((r[tw][0] & 0xFFFFu) | (r[tw][4] & 0xFFFF0000u)) : 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) dd[u] = dpk;
            xpose4(v0);
            xpose4(v1);
            xpose4(dd);  // dd[s] = scales of lane group s's pair
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
                for (int R = 0; R < 2; ++R) {
                    const int blk = 2 * s2 + R;  // block index within the step
                    const half8_t ah = *reinterpret_cast<const half8_t*>(xa + blk * 2048);
                    const half8_t al = *reinterpret_cast<const half8_t*>(xa + blk * 2048 + 1024);
                    const half8_t bq = q4_codes_f16(R ? v1[s2] : v0[s2]);
                    f32x4_t cc = {0.f, 0.f, 0.f, 0.f};
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq, cc, 0, 0, 0);
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bq, cc, 0, 0, 0);
                    const float d = R ? half_hi(dd[s2]) : half_lo(dd[s2]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) cacc[tw][i] = fmaf(d, cc[i], cacc[tw][i]);
                }
            }
        }
        if ((step + 1) % steps_per_chunk == 0 || step + 1 == nsteps) {
            // fold this chunk's partial sums with the chunk's activation scales
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sc = s_scale[buf][4 * G + i];
#pragma unroll
                for (int tw = 0; tw < TW; ++tw) {
                    acc[tw][i] = fmaf(sc, cacc[tw][i], acc[tw][i]);
                    cacc[tw][i] = 0.f;
                }
            }
        }
    };

    for (int step = 0; step < nsteps; step += 2) {
        // stage the next chunk while this one is consumed
        const int c = step / steps_per_chunk;
        if (step % steps_per_chunk == 0 && c + 1 < nchunks) stage(c + 1, (c + 1) & 1);
        compute(step, b0);
        if (step + 2 < nsteps) issue(step + 2, b0);
        if (step + 1 < nsteps) {
            compute(step + 1, b1);
            if (step + 3 < nsteps) issue(step + 3, b1);
        }
        if ((step + 2) % steps_per_chunk == 0) __syncthreads();  // chunk c consumed, c + 1 staged
    }
    // lane (G, j) holds rows 4G..4G+3 of activation rows, weight row j of each tile
#pragma unroll
    for (int tw = 0; tw < TW; ++tw) {
        const long row = row_base + tw * 16 + j;
        if (row < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * G + i;
                if (m < M) Y[(size_t)m * ldy + row] = acc[tw][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// M = 2..16, second form: the activations are converted once per call by a
// small pre-pass into a stream-ordered scratch buffer, already in A-operand
// order, and every wave loads its A operands straight from there (L2
// resident, 1 KB contiguous per block and piece), so the main kernel has no
// LDS staging and no barriers in its K loop.
//
// Pre-pass (one workgroup per activation row m < 16): s_m = the power of two
// that puts max_k |x[m, k]| in [2^14, 2^15) (fp16 range; rows past M are
// zero), then x * 2^s_m = hi + lo with hi, lo fp16. Scratch layout per block
// b: piece p (hi, lo) x row m x slice G x 8 halves = 2 KB, then 16 floats
// with 2^-s_m.
//
// Main kernel: a workgroup has S * WR waves; wave (s, rw) owns TW tiles of
// 16 weight rows and the s-th of S segments of each row's block pairs; the S
// partial sums meet in LDS once at the end.
// ---------------------------------------------------------------------------
// One workgroup per activation row m < 16 (1024 threads, up to XP_PER
// elements per thread held in registers, so x is read once).
constexpr int XP_THREADS = 1024, XP_PER = 16;
constexpr int XP_KMAX = XP_THREADS * XP_PER;

__global__ __launch_bounds__(XP_THREADS) void k_xprep(const float* __restrict__ X, size_t ldx, int M, int K,
                                                      uint8_t* __restrict__ xa, int* __restrict__ zero_me,
                                                      int n_zero) {
    __shared__ float red[XP_THREADS / 64];
    const int m = blockIdx.x;  // 0..15
    for (int i = threadIdx.x; i < n_zero && m == 0; i += XP_THREADS) zero_me[i] = 0;
    float v[XP_PER];
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < XP_PER; ++e) {
        const int k = threadIdx.x + e * XP_THREADS;
        v[e] = (m < M && k < K) ? X[(size_t)m * ldx + k] : 0.f;
        mx = fmaxf(mx, fabsf(v[e]));
    }
    mx = wave_max(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < XP_THREADS / 64; ++w) mx = fmaxf(mx, red[w]);
    int sh = 0;
    if (mx > 0.f && mx <= 3.4e38f) {
        int ex;
        frexpf(mx, &ex);
        sh = 15 - ex;
        sh = sh > 126 ? 126 : (sh < -126 ? -126 : sh);
    }
    const size_t nb = (size_t)K / 32;
    if (threadIdx.x == 0) reinterpret_cast<float*>(xa + nb * 2048)[m] = ldexpf(1.f, -sh);
#pragma unroll
    for (int e = 0; e < XP_PER; ++e) {
        const int k = threadIdx.x + e * XP_THREADS;
        if (k < K) {
            const float t = ldexpf(v[e], sh);
            const _Float16 h = (_Float16)t;
            const _Float16 l = (_Float16)(t - (float)h);
            const int el = k & 31, g = (el & 15) >> 2;
            uint8_t* rec = xa + (size_t)(k >> 5) * 2048 + m * 64 + g * 16 + slice_pos(el) * 2;
            *reinterpret_cast<_Float16*>(rec) = h;
            *reinterpret_cast<_Float16*>(rec + 1024) = l;
        }
    }
}

struct MmPlan {
    int S, seg, WR;
};

template <int TW>
__global__ __launch_bounds__(512) void k_mm2(const uint8_t* __restrict__ W, size_t ldw, const uint8_t* __restrict__ xa,
                                             float* __restrict__ Y, size_t ldy, int M, int N, int K, MmPlan plan) {
    __shared__ f32x4_t red[8][TW][64];
    const int S = plan.S, seg = plan.seg;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sgi = wave % S, rw = wave / S;
    const int G = lane >> 4, j = lane & 15;
    const int P = K >> 6;
    const int p0 = sgi * seg;
    const int p1 = p0 + seg < P ? p0 + seg : P;
    const int nsteps = (seg + 3) >> 2;
    const long row_base = ((long)blockIdx.x * plan.WR + rw) * 16 * TW;

    auto issue = [&](int t, uint32_t (&b)[TW][9]) {
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
            long row = row_base + tw * 16 + j;
            row = row < N ? row : N - 1;
            int q = p0 + 4 * t + G;
            q = q < p1 ? q : p1 - 1;
            q = q > 0 ? q : 0;
            load_pair<9>(W + row * ldw + (size_t)q * 36, b[tw]);
        }
    };
    f32x4_t acc[TW];
#pragma unroll
    for (int tw = 0; tw < TW; ++tw) acc[tw] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    const uint8_t* xl = xa + j * 64 + G * 16;  // this lane's A slice within a block record

    auto compute = [&](int t, uint32_t (&r)[TW][9]) {
        const int qbase = p0 + 4 * t;  // pair of lane group 0
        uint32_t v0[TW][4], v1[TW][4], dd[TW][4];
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
            const bool valid = qbase + G < p1;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v0[tw][u] = __builtin_amdgcn_alignbyte(r[tw][u + 1], r[tw][u], 2);
                v1[tw][u] = r[tw][5 + u];
            }
            const uint32_t dpk = valid ? ((r[tw][0] & 0xFFFFu) | (r[tw][4] & 0xFFFF0000u)) : 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) dd[tw][u] = dpk;
            xpose4(v0[tw]);
            xpose4(v1[tw]);
            xpose4(dd[tw]);
        }
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                int blk = 2 * (qbase + s2) + R;  // global block index
                blk = blk < 2 * P ? blk : 2 * P - 1;
                const uint8_t* rec = xl + (size_t)blk * 2048;
                const half8_t ah = *reinterpret_cast<const half8_t*>(rec);
                const half8_t al = *reinterpret_cast<const half8_t*>(rec + 1024);
#pragma unroll
                for (int tw = 0; tw < TW; ++tw) {
                    const half8_t bq = q4_codes_f16(R ? v1[tw][s2] : v0[tw][s2]);
                    f32x4_t cc = {0.f, 0.f, 0.f, 0.f};
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq, cc, 0, 0, 0);
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bq, cc, 0, 0, 0);
                    const float d = R ? half_hi(dd[tw][s2]) : half_lo(dd[tw][s2]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[tw][i] = fmaf(d, cc[i], acc[tw][i]);
                }
            }
        }
    };

    uint32_t b0[TW][9], b1[TW][9];
    if (nsteps > 0) issue(0, b0);
    if (nsteps > 1) issue(1, b1);
    for (int t = 0; t < nsteps; t += 2) {
        compute(t, b0);
        if (t + 2 < nsteps) issue(t + 2, b0);
        if (t + 1 < nsteps) {
            compute(t + 1, b1);
            if (t + 3 < nsteps) issue(t + 3, b1);
        }
    }
    const float* rscale = reinterpret_cast<const float*>(xa + (size_t)(K / 32) * 2048);
    if (S > 1) {
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) red[wave][tw][lane] = acc[tw];
        __syncthreads();
        if (sgi != 0) return;
        for (int q2 = 1; q2 < S; ++q2)
#pragma unroll
            for (int tw = 0; tw < TW; ++tw) acc[tw] += red[wave + q2][tw][lane];
    }
#pragma unroll
    for (int tw = 0; tw < TW; ++tw) {
        const long row = row_base + tw * 16 + j;
        if (row < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * G + i;
                if (m < M) Y[(size_t)m * ldy + row] = acc[tw][i] * rscale[m];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// M = 2..16, third form: the eight waves of a workgroup work on eight
// different 16-row tiles (TW tiles each) over the same K range, so they share
// the A operands, which are copied chunk by chunk (512 columns = 32 KB) from
// the converted activations into double-buffered LDS: the next chunk is
// loaded into registers while the current one is consumed and written to the
// other buffer before the one barrier per chunk. K is split over
// grid.y workgroups when there are too few tiles to fill the chip; their
// partial sums go to scratch and the last workgroup of a tile group (by an
// atomic arrival count) adds them in segment order, so the result does not
// depend on timing.
// ---------------------------------------------------------------------------
constexpr int MM3_WAVES = 8;

template <int TW>
__global__ __launch_bounds__(MM3_WAVES * 64) void k_mm3(const uint8_t* __restrict__ W, size_t ldw,
                                                        const uint8_t* __restrict__ xa, float* __restrict__ Y,
                                                        size_t ldy, int M, int N, int K, int chunks_per_seg,
                                                        float* __restrict__ part, int* __restrict__ arrive) {
    extern __shared__ __align__(16) uint8_t smem[];  // 2 x 32 KB A chunks
    __shared__ int s_last;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
    const int G = lane >> 4, j = lane & 15;
    const int P = K >> 6;
    const int nchunks = (K + MM_KC - 1) / MM_KC;
    const int S = gridDim.y, sgi = blockIdx.y;
    const int c0 = sgi * chunks_per_seg;
    const int c1 = c0 + chunks_per_seg < nchunks ? c0 + chunks_per_seg : nchunks;
    const long row_base = ((long)blockIdx.x * MM3_WAVES + wave) * 16 * TW;
    const size_t xa_bytes = (size_t)(K / 32) * 2048;

    // A chunk c: 16 blocks x 2 KB, contiguous in xa; 512 threads x 4 x 16 B.
    typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));
    u32x4a stg[4];
    auto fetch_a = [&](int c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            size_t off = (size_t)c * MM_CHUNK_BYTES + (size_t)(i * MM3_WAVES * 64 + tid) * 16;
            off = off < xa_bytes ? off : 0;  // the tail of the last chunk is never read
            stg[i] = *reinterpret_cast<const u32x4a*>(xa + off);
        }
    };
    auto put_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4a*>(smem + buf * MM_CHUNK_BYTES + (i * MM3_WAVES * 64 + tid) * 16) = stg[i];
    };

    auto issue = [&](int step, uint32_t (&b)[TW][9]) {
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
            long row = row_base + tw * 16 + j;
            row = row < N ? row : N - 1;
            int q = step * 4 + G;
            q = q < P ? q : P - 1;
            load_pair<9>(W + row * ldw + (size_t)q * 36, b[tw]);
        }
    };
    f32x4_t acc[TW];
#pragma unroll
    for (int tw = 0; tw < TW; ++tw) acc[tw] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int step, const uint8_t* xbuf, uint32_t (&r)[TW][9]) {
        const int qbase = step * 4;
        const bool valid = qbase + G < P;
        uint32_t v0[TW][4], v1[TW][4], dd[TW][4];
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v0[tw][u] = __builtin_amdgcn_alignbyte(r[tw][u + 1], r[tw][u], 2);
                v1[tw][u] = r[tw][5 + u];
            }
            const uint32_t dpk = valid ? ((r[tw][0] & 0xFFFFu) | (r[tw][4] & 0xFFFF0000u)) : 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) dd[tw][u] = dpk;
            xpose4(v0[tw]);
            xpose4(v1[tw]);
            xpose4(dd[tw]);
        }
        const uint8_t* xl = xbuf + (step & 1) * 8 * 2048 + j * 64 + G * 16;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                const uint8_t* rec = xl + (2 * s2 + R) * 2048;
                const half8_t ah = *reinterpret_cast<const half8_t*>(rec);
                const half8_t al = *reinterpret_cast<const half8_t*>(rec + 1024);
#pragma unroll
                for (int tw = 0; tw < TW; ++tw) {
                    const half8_t bq = q4_codes_f16(R ? v1[tw][s2] : v0[tw][s2]);
                    f32x4_t cc = {0.f, 0.f, 0.f, 0.f};
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bq, cc, 0, 0, 0);
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bq, cc, 0, 0, 0);
                    const float d = R ? half_hi(dd[tw][s2]) : half_lo(dd[tw][s2]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[tw][i] = fmaf(d, cc[i], acc[tw][i]);
                }
            }
        }
    };

    // Two steps (256 columns each) per chunk; W loads two steps ahead.
    uint32_t b0[TW][9], b1[TW][9];
    const int st0 = c0 * 2, st1 = c1 * 2;
    if (st0 < st1) {
        issue(st0, b0);
        issue(st0 + 1, b1);
        fetch_a(c0);
        put_a(0);
    }
    __syncthreads();
    for (int c = c0; c < c1; ++c) {
        const int buf = (c - c0) & 1;
        if (c + 1 < c1) fetch_a(c + 1);
        const uint8_t* xbuf = smem + buf * MM_CHUNK_BYTES;
        compute(2 * c, xbuf, b0);
        if (2 * c + 2 < st1) issue(2 * c + 2, b0);
        compute(2 * c + 1, xbuf, b1);
        if (2 * c + 3 < st1) issue(2 * c + 3, b1);
        if (c + 1 < c1) put_a(buf ^ 1);
        __syncthreads();
    }

    const float* rscale = reinterpret_cast<const float*>(xa + xa_bytes);
    if (S > 1) {
        // publish this segment's partial tile sums, then the last arrival adds them
        float* mine = part + ((size_t)sgi * gridDim.x + blockIdx.x) * (MM3_WAVES * TW * 64 * 4);
#pragma unroll
        for (int tw = 0; tw < TW; ++tw)
            *reinterpret_cast<f32x4_t*>(mine + ((wave * TW + tw) * 64 + lane) * 4) = acc[tw];
        __threadfence();
        __syncthreads();
        if (tid == 0) s_last = atomicAdd(&arrive[blockIdx.x], 1) == S - 1;
        __syncthreads();
        if (!s_last) return;
        __threadfence();
#pragma unroll
        for (int tw = 0; tw < TW; ++tw) acc[tw] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        for (int q2 = 0; q2 < S; ++q2) {
            const float* pp = part + ((size_t)q2 * gridDim.x + blockIdx.x) * (MM3_WAVES * TW * 64 * 4);
#pragma unroll
            for (int tw = 0; tw < TW; ++tw)
                acc[tw] += __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pp + ((wave * TW + tw) * 64 + lane) * 4));
        }
    }
#pragma unroll
    for (int tw = 0; tw < TW; ++tw) {
        const long row = row_base + tw * 16 + j;
        if (row < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * G + i;
                if (m < M) Y[(size_t)m * ldy + row] = acc[tw][i] * rscale[m];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Generic kernel: any qtype, 1..MT rows of X, 2-byte alignment, any K % 32.
// One wave per weight row (4 waves per workgroup), one block per lane step.
// ---------------------------------------------------------------------------
template <int QT>
__device__ __forceinline__ void decode_block_generic(const uint8_t* bp, float& d, float* c) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(bp);
    d = (float)__builtin_bit_cast(_Float16, h[0]);
    if constexpr (QT == QMV_Q4_0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t v = h[1 + i];
            c[2 * i] = (float)((int)(v & 0xF) - 8);
            c[2 * i + 16] = (float)((int)((v >> 4) & 0xF) - 8);
            c[2 * i + 1] = (float)((int)((v >> 8) & 0xF) - 8);
            c[2 * i + 17] = (float)((int)((v >> 12) & 0xF) - 8);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t v = h[1 + i];
            c[2 * i] = (float)(int8_t)(v & 0xFF);
            c[2 * i + 1] = (float)(int8_t)(v >> 8);
        }
    }
}

template <int MT>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// y_m = sum over row `wr` (K/32 blocks) of w * X[xrow[m]], m < M; lane-partial.
template <int QT, int MT>
__device__ __forceinline__ void generic_row(const uint8_t* __restrict__ wr, const float* __restrict__ X,
                                            const size_t* xoff, int M, int K, int lane, float* acc) {
    constexpr int BB = block_bytes(QT);
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
    const int nb = K / QK;
    for (int b = lane; b < nb; b += 64) {
        float d, c[32];
        decode_block_generic<QT>(wr + (size_t)b * BB, d, c);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < M) {
                const float* xp = X + xoff[m] + (size_t)b * QK;
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s0 = fmaf(c[i], xp[i], s0);
                    s1 = fmaf(c[16 + i], xp[16 + i], s1);
                }
                acc[m] = fmaf(d, s0 + s1, acc[m]);
            }
        }
    }
}

template <int QT, int MT>
__global__ __launch_bounds__(256) void k_generic(const uint8_t* __restrict__ W, size_t ldw,
                                                 const float* __restrict__ X, size_t ldx, float* __restrict__ Y,
                                                 size_t ldy, int M, int N, int K) {
    const int lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= N) return;
    size_t xoff[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xoff[m] = (size_t)m * ldx;
    float acc[MT];
    generic_row<QT, MT>(W + row * ldw, X, xoff, M, K, lane, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (m < M) {
            float s = wave_sum<64>(acc[m]);
            if (lane == 0) Y[(size_t)m * ldy + row] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// Expert-indexed kernel.
// grid = (row tiles, pairs). Workgroup (tile, p): e = ids[p].
//  * e >= n_experts: rows of Y[p] in the tile get NaN, *err_flag = 1.
//  * an earlier pair q < p has the same e: exit (that pair's workgroup
//    covers p too).
//  * otherwise gather every pair q >= p with ids[q] == e (in order) and
//    compute their rows of this tile, streaming expert e's rows once.
// ---------------------------------------------------------------------------
constexpr int ID_MAX_LIST = 1024;  // pairs one leader can serve in one pass

template <int QT, int LPR, int RPT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_id(const uint8_t* __restrict__ W, size_t estride, size_t ldw,
                                                   int n_experts, const float* __restrict__ X, size_t ldx,
                                                   const uint32_t* __restrict__ ids, int n_pairs, int top_k,
                                                   float* __restrict__ Y, size_t ldy, int N, int K,
                                                   const float* __restrict__ escale, int* __restrict__ err_flag,
                                                   int fast) {
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS_PER_WG = GROUPS * RPT * WAVES;
    __shared__ int s_list[ID_MAX_LIST];
    __shared__ int s_count;
    __shared__ int s_dup;
    extern __shared__ __align__(16) float xs[];

    const int p = blockIdx.y;
    const uint32_t e = ids[p];
    const long tile_row0 = (long)blockIdx.x * ROWS_PER_WG;
    const int tid = threadIdx.x;

    if (e >= (uint32_t)n_experts) {
        for (long n = tile_row0 + tid; n < tile_row0 + ROWS_PER_WG && n < N; n += blockDim.x)
            Y[(size_t)p * ldy + n] = __builtin_nanf("");
        if (tid == 0 && err_flag) *err_flag = 1;
        return;
    }
    if (tid == 0) { s_dup = 0; s_count = 0; }
    __syncthreads();
    for (int q = tid; q < p; q += blockDim.x)
        if (ids[q] == e) s_dup = 1;
    __syncthreads();
    if (s_dup) return;
    // Ordered gather of the pairs served here (wave 0, 64 ids per step).
    if (tid < 64) {
        int base = 0;
        for (int q0 = p; q0 < n_pairs; q0 += 64) {
            const int q = q0 + tid;
            const bool hit = q < n_pairs && ids[q] == e;
            const uint64_t mask = __ballot(hit);
            const int pos = base + __popcll(mask & ((1ull << tid) - 1ull));
            if (hit && pos < ID_MAX_LIST) s_list[pos] = q;
            base += __popcll(mask);
        }
        if (tid == 0) s_count = base;
    }
    __syncthreads();
    const int count = s_count;
    const uint8_t* We = W + (size_t)e * estride;

    if (count == 1 && fast) {
        const int t = p / top_k;
        const float sc = (escale ? escale[e] : 1.f) * PairTraits<QT>::OUT_SCALE;
        m1_stream<QT, LPR, RPT, WAVES>(We, ldw, X + (size_t)t * ldx, Y + (size_t)p * ldy, N, K, blockIdx.x,
                                       gridDim.x, sc, xs);
        return;
    }
    // General case: one wave per row, up to 16 pairs per pass.
    const int lane = tid & 63, wave = tid >> 6;
    const float sc = escale ? escale[e] : 1.f;
    const int served = count < ID_MAX_LIST ? count : ID_MAX_LIST;
    for (int c0 = 0; c0 < served; c0 += 16) {
        const int M = served - c0 < 16 ? served - c0 : 16;
        size_t xoff[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) xoff[m] = (size_t)(s_list[c0 + (m < M ? m : 0)] / top_k) * ldx;
        for (long n = tile_row0 + wave; n < tile_row0 + ROWS_PER_WG && n < N; n += WAVES) {
            float acc[16];
            generic_row<QT, 16>(We + n * ldw, X, xoff, M, K, lane, acc);
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                if (m < M) {
                    float s = wave_sum<64>(acc[m]);
                    if (lane == 0) Y[(size_t)s_list[c0 + m] * ldy + n] = s * sc;
                }
            }
        }
    }
    // The host launches at most ID_MAX_LIST pairs at a time, so the list
    // always holds every pair of this launch that selects e.
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int KMAX_FAST = 15360;     // x staged in <= 64 KiB of LDS
constexpr int KMAX_FAST_ID = 14336;  // same, next to the id kernel's pair list

constexpr size_t LDS_PER_CU = 160 * 1024;  // gfx950

// Compute units of the current device (cached per device id).
int num_cus() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev < 64) cache[dev] = n;
    return n;
}

// Lanes per row: the largest power of two (<= 64) whose lane utilisation
// P / (LPR * ceil(P / LPR)) is within 5% of the best one, so long rows keep
// a full wave on one row and short rows still use every lane.
int pick_lpr(int P) {
    const int cands[] = {64, 32, 16, 8, 4};
    double eff[5], best = 0;
    for (int i = 0; i < 5; ++i) {
        const int l = cands[i];
        eff[i] = (double)P / ((double)l * ((P + l - 1) / l));
        if (eff[i] > best) best = eff[i];
    }
    for (int i = 0; i < 5; ++i)
        if (eff[i] >= best * 0.95) return cands[i];
    return 4;
}

struct M1Cfg {
    int lpr, rpt, waves, wgs_per_cu;
};

M1Cfg pick_m1(int N, int K) {
    M1Cfg c;
    c.lpr = pick_lpr(K / 64);
    c.rpt = 1;
    c.waves = 8;
    c.wgs_per_cu = 2;
    (void)N;
    return c;
}

template <int QT, int LPR, int RPT, int WAVES>
int launch_m1_t(const uint8_t* W, size_t ldw, const float* X, float* Y, int N, int K, int wgs_per_cu,
                hipStream_t st) {
    constexpr int ROWS = (64 / LPR) * RPT * WAVES;
    const long tiles = ((long)N + ROWS - 1) / ROWS;
    const size_t lds = xs_bytes(K);
    long per_cu = (long)(LDS_PER_CU / (lds ? lds : 1));
    per_cu = per_cu < 1 ? 1 : (per_cu < wgs_per_cu ? per_cu : wgs_per_cu);
    long grid = (long)num_cus() * per_cu;
    grid = grid < tiles ? grid : tiles;
    hipLaunchKernelGGL((k_m1<QT, LPR, RPT, WAVES>), dim3((unsigned)grid), dim3(WAVES * 64), lds, st, W, ldw, X, Y, N,
                       K);
    return check_launch("qmv m1 kernel");
}

template <int QT>
int launch_m1(const uint8_t* W, size_t ldw, const float* X, float* Y, int N, int K, hipStream_t st) {
    const M1Cfg c = pick_m1(N, K);
#define QMV_M1_CASE(L, R, WV) \
    if (c.lpr == L && c.rpt == R && c.waves == WV) return launch_m1_t<QT, L, R, WV>(W, ldw, X, Y, N, K, c.wgs_per_cu, st);
    QMV_M1_CASE(64, 1, 8) QMV_M1_CASE(32, 1, 8) QMV_M1_CASE(16, 1, 8) QMV_M1_CASE(8, 1, 8) QMV_M1_CASE(4, 1, 8)
#undef QMV_M1_CASE
    return fail(QMV_EINVAL, "internal: no m1 kernel for lpr=%d rpt=%d waves=%d", c.lpr, c.rpt, c.waves);
}

// Plan for the x-stationary kernel: lanes per row and K segments.
struct M1xCfg {
    int lpr, rpt, wr, wgs_per_cu;
};

XsPlan make_plan(int P, int lpr, int wr) {
    XsPlan pl;
    pl.S = (P + lpr - 1) / lpr;
    pl.seg = (P + pl.S - 1) / pl.S;
    pl.WR = wr;
    while (pl.S * pl.WR > 8 && pl.WR > 1) --pl.WR;
    return pl;
}

template <int QT, int LPR, int RPT>
int launch_m1x_t(const uint8_t* W, size_t ldw, const float* X, float* Y, int N, int K, int wr, int wgs_per_cu,
                 float out_scale, hipStream_t st) {
    const XsPlan pl = make_plan(K / 64, LPR, wr);
    if (pl.S > 8) return fail(QMV_EINVAL, "internal: K=%d too long for the x-stationary kernel", K);
    const int rows_step = pl.WR * (64 / LPR) * RPT;
    const long nsteps = ((long)N + rows_step - 1) / rows_step;
    long grid = (long)num_cus() * wgs_per_cu;
    grid = grid < nsteps ? grid : nsteps;
    hipLaunchKernelGGL((k_m1x<QT, LPR, RPT>), dim3((unsigned)grid), dim3(64 * pl.S * pl.WR), 0, st, W, ldw, X, Y, N,
                       K, pl, out_scale);
    return check_launch("qmv m1x kernel");
}

int launch_m1h(const uint8_t* W, size_t ldw, const float* X, float* Y, int N, int K, int target_wpc, int wgs_per_cu,
               int force_S, hipStream_t st) {
    const int ncu = num_cus();
    MhPlan pl = make_mh_plan(N, K, ncu, target_wpc);
    if (force_S > 0) {
        pl.S = force_S;
        pl.seg = (K / 64 + force_S - 1) / force_S;
        pl.WR = force_S >= 8 ? 1 : 8 / force_S;
    }
    const long ntiles = ((long)N + 15) / 16;
    long grid = (long)ncu * wgs_per_cu;
    const long need = (ntiles + pl.WR - 1) / pl.WR;
    grid = grid < need ? grid : need;
    const size_t lds = (size_t)(K / 32) * 128;
    hipLaunchKernelGGL(k_m1h, dim3((unsigned)grid), dim3(64 * pl.S * pl.WR), lds, st, W, ldw, X, Y, N, K, pl, 1.0f);
    return check_launch("qmv m1h kernel");
}

// Lanes per row for the batched kernel: favour more rows in flight (more
// waves) over lane utilisation, since these products are latency-bound: the
// largest power of two not above 4/3 of the pairs per row.
int m1b_lpr(int P) {
    int l = 64;
    while (l > 4 && 3 * l > 4 * P) l >>= 1;
    return l;
}

// Problems a batched M = 1 launch can take (checked by the caller).
bool m1b_eligible(const uint8_t* W, size_t ldw, const float* x, int K) {
    return K > 0 && K % 64 == 0 && K <= KMAX_FAST && ((uintptr_t)W & 3) == 0 && (ldw & 3) == 0 &&
           ((uintptr_t)x & 3) == 0;
}

// Launch the batched M = 1 kernel over n problems (n <= MAXB), all eligible.
// wgs_per_cu and waves are tuning knobs (0 = default).
template <int QT>
int launch_m1b(const M1Prob* probs, int n, int wgs_per_cu, int waves, hipStream_t st) {
    if (waves == 0) waves = 8;
    if (wgs_per_cu == 0) wgs_per_cu = 2;
    M1Batch B;
    B.n = 0;
    size_t lds = 0;
    double total = 0;
    const int bb = block_bytes(QT);
    for (int i = 0; i < n; ++i) total += (double)probs[i].N * (probs[i].K / QK) * bb;
    for (int i = 0; i < n; ++i) lds = xs_bytes(probs[i].K) > lds ? xs_bytes(probs[i].K) : lds;
    long per_cu = (long)(LDS_PER_CU / (lds ? lds : 1));
    per_cu = per_cu < 1 ? 1 : (per_cu < wgs_per_cu ? per_cu : wgs_per_cu);
    const long budget = (long)num_cus() * per_cu;
    long wg = 0;
    for (int i = 0; i < n; ++i) {
        M1Prob q = probs[i];
        q.lpr = pick_lpr(q.K / 64);
        const long rows = (long)(64 / q.lpr) * waves;  // rows per tile
        const long tiles = ((long)q.N + rows - 1) / rows;
        const double bytes = (double)q.N * (q.K / QK) * bb;
        long nwg = (long)(budget * bytes / total + 0.5);
        nwg = nwg < 1 ? 1 : (nwg > tiles ? tiles : nwg);
        q.wg0 = (int)wg;
        q.nwg = (int)nwg;
        wg += nwg;
        B.p[B.n++] = q;
    }
    if (wg > 0x7FFFFFFF) return fail(QMV_EINVAL, "N too large");
    if (waves == 16)
        hipLaunchKernelGGL((k_m1b<QT, 16>), dim3((unsigned)wg), dim3(1024), lds, st, B);
    else if (waves == 4)
        hipLaunchKernelGGL((k_m1b<QT, 4>), dim3((unsigned)wg), dim3(256), lds, st, B);
    else
        hipLaunchKernelGGL((k_m1b<QT, 8>), dim3((unsigned)wg), dim3(512), lds, st, B);
    return check_launch("qmv batched m1 kernel");
}

bool mo_eligible(const uint8_t* W, size_t ldw, const float* x, int K) {
    return K > 0 && K % 64 == 0 && K <= MO_KMAX && ((uintptr_t)W & 3) == 0 && (ldw & 3) == 0 &&
           ((uintptr_t)x & 3) == 0;
}

// Launch the one-shot M = 1 kernel over n problems (all mo_eligible).
// Knobs (0 = default): MAXI (4 or 8), target waves per CU.
template <int QT>
int launch_m1o(const M1Prob* probs, int n, int maxi, int wpc, hipStream_t st) {
    if (maxi == 0) maxi = 4;
    if (wpc <= 0) wpc = 16;
    const int ncu = num_cus();
    const int bb = block_bytes(QT);
    double total = 0;
    for (int i = 0; i < n; ++i) total += (double)probs[i].N * (probs[i].K / QK) * bb;
    OsBatch B;
    B.n = 0;
    long wg = 0;
    size_t lds = 0;
    for (int i = 0; i < n; ++i) {
        OsProb q;
        q.W = probs[i].W;
        q.x = probs[i].x;
        q.y = probs[i].y;
        q.ldw = probs[i].ldw;
        q.N = probs[i].N;
        q.K = probs[i].K;
        const int P = q.K / 64;
        int S = 1;
        while (S * 64 < P) S *= 2;
        int lpr = 4;
        if (S > 1) {
            lpr = 64;
        } else {
            while (lpr < P) lpr *= 2;
        }
        q.lpr = lpr;
        q.S = S;
        const int R = MO_WAVES / S;
        const long RG = ((long)q.N + 64 / lpr - 1) / (64 / lpr);
        const long tr_min = (RG + maxi - 1) / maxi;
        const double bytes = (double)q.N * (q.K / QK) * bb;
        long tr = (long)((double)ncu * wpc / S * bytes / total + 0.5);
        tr = tr > RG ? RG : tr;
        tr = tr < tr_min ? tr_min : tr;
        tr = tr < 1 ? 1 : tr;
        const long nwg = (tr + R - 1) / R;
        q.wg0 = (int)wg;
        q.nwg = (int)nwg;
        wg += nwg;
        B.p[B.n++] = q;
        const size_t l = xs_bytes(q.K);
        lds = l > lds ? l : lds;
    }
    if (wg > 0x7FFFFFFF) return fail(QMV_EINVAL, "N too large");
    if (maxi == 8)
        hipLaunchKernelGGL((k_m1o<QT, 8>), dim3((unsigned)wg), dim3(MO_WAVES * 64), lds, st, B);
    else
        hipLaunchKernelGGL((k_m1o<QT, 4>), dim3((unsigned)wg), dim3(MO_WAVES * 64), lds, st, B);
    return check_launch("qmv one-shot m1 kernel");
}

bool mq_eligible(const uint8_t* W, size_t ldw, const float* x, int K) {
    return K > 0 && K % 64 == 0 && K <= MQ_KMAX && ((uintptr_t)W & 3) == 0 && (ldw & 3) == 0 &&
           ((uintptr_t)x & 3) == 0;
}

// Segments per tile: enough (tile, segment) waves for target_waves, each
// segment keeping at least 8 pairs (two steps), at most 16 segments.
int mq_segments(long ntiles, int P, long target_waves) {
    int S = 1;
    while (S < 16 && ntiles * S < target_waves && (P + 2 * S - 1) / (2 * S) >= 8) S *= 2;
    return S;
}

// Launch the block-diagonal matrix-core M = 1 kernel over n Q4_0 problems
// (n <= MAXB, all mq_eligible). Tuning knobs (0 = default): target waves per
// CU, workgroups per CU, forced segment count.
int launch_m1q(const M1Prob* probs, int n, int target_wpc, int wgs_per_cu, int force_S, hipStream_t st) {
    const int ncu = num_cus();
    if (target_wpc <= 0) target_wpc = 12;
    int S[MAXB];
    long ntg[MAXB];
    double bytes[MAXB], total = 0;
    int waves = 8;
    size_t lds = 0;
    for (int i = 0; i < n; ++i) {
        const long ntiles = ((long)probs[i].N + 15) / 16;
        const int P = probs[i].K / 64;
        S[i] = force_S ? force_S : mq_segments(ntiles, P, (long)ncu * target_wpc);
        if (S[i] != 1 && S[i] != 2 && S[i] != 4 && S[i] != 8 && S[i] != 16)
            return fail(QMV_EINVAL, "internal: segment count %d", S[i]);
        waves = S[i] > waves ? S[i] : waves;
        const size_t l = mq_lds_bytes(probs[i].K);
        lds = l > lds ? l : lds;
        bytes[i] = (double)probs[i].N * (probs[i].K / QK) * 18;
        total += bytes[i];
    }
    long sum_ntg = 0;
    for (int i = 0; i < n; ++i) {
        const long ntiles = ((long)probs[i].N + 15) / 16;
        const int T = waves / S[i];
        ntg[i] = (ntiles + T - 1) / T;
        sum_ntg += ntg[i];
    }
    const size_t red = 2 * (size_t)waves * 16 * sizeof(float);
    if (wgs_per_cu <= 0) {
        const long by_lds = (long)(LDS_PER_CU / (lds + red));
        const long by_waves = 32 / waves;
        wgs_per_cu = (int)(by_lds < by_waves ? by_lds : by_waves);
        if (wgs_per_cu < 1) wgs_per_cu = 1;
    }
    const long budget = (long)ncu * wgs_per_cu;
    MqBatch B;
    B.n = 0;
    long wg = 0;
    for (int i = 0; i < n; ++i) {
        MqProb q;
        q.W = probs[i].W;
        q.x = probs[i].x;
        q.y = probs[i].y;
        q.ldw = probs[i].ldw;
        q.N = probs[i].N;
        q.K = probs[i].K;
        q.S = S[i];
        q.segP = (q.K / 64 + S[i] - 1) / S[i];
        long nwg = sum_ntg <= budget ? ntg[i] : (long)(budget * bytes[i] / total + 0.5);
        nwg = nwg < 1 ? 1 : (nwg > ntg[i] ? ntg[i] : nwg);
        q.wg0 = (int)wg;
        q.nwg = (int)nwg;
        wg += nwg;
        B.p[B.n++] = q;
    }
    if (wg > 0x7FFFFFFF) return fail(QMV_EINVAL, "N too large");
    if (waves == 16)
        hipLaunchKernelGGL((k_m1q<16>), dim3((unsigned)wg), dim3(1024), lds, st, B);
    else
        hipLaunchKernelGGL((k_m1q<8>), dim3((unsigned)wg), dim3(512), lds, st, B);
    return check_launch("qmv matrix-core m1 kernel");
}

// M = 2..16 on the matrix cores (Q4_0, K % 64 == 0, 4-byte aligned rows).
template <int WAVES, int TW>
int launch_mm_t(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
                hipStream_t st) {
    const long rows_wg = 16L * TW * WAVES;
    const long grid = ((long)N + rows_wg - 1) / rows_wg;
    if (grid > 0x7FFFFFFF) return fail(QMV_EINVAL, "N too large");
    hipLaunchKernelGGL((k_mm<WAVES, TW>), dim3((unsigned)grid), dim3(WAVES * 64), 2 * MM_CHUNK_BYTES, st, W, ldw, X,
                       ldx, Y, ldy, M, N, K);
    return check_launch("qmv mfma kernel");
}

int launch_mm(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
              int waves, int tw, hipStream_t st) {
    if (waves == 0) {
        // enough workgroups to cover the chip; more rows per wave when there are plenty
        const long tiles = ((long)N + 15) / 16;
        waves = 4;
        tw = tiles >= 4L * 4 * num_cus() ? 2 : 1;
    }
    if (waves == 4 && tw == 1) return launch_mm_t<4, 1>(W, ldw, X, ldx, Y, ldy, M, N, K, st);
    if (waves == 4 && tw == 2) return launch_mm_t<4, 2>(W, ldw, X, ldx, Y, ldy, M, N, K, st);
    if (waves == 8 && tw == 1) return launch_mm_t<8, 1>(W, ldw, X, ldx, Y, ldy, M, N, K, st);
    if (waves == 8 && tw == 2) return launch_mm_t<8, 2>(W, ldw, X, ldx, Y, ldy, M, N, K, st);
    return fail(QMV_EINVAL, "internal: no mfma kernel for waves=%d tw=%d", waves, tw);
}

// M = 2..16 with the activation pre-pass; returns QMV_EUNSUPPORTED (nothing
// enqueued) when the scratch buffer cannot be allocated, so the caller can
// fall back to the staging kernel.
int launch_mm2(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
               int force_S, int force_tw, hipStream_t st) {
    if (K > XP_KMAX) return QMV_EUNSUPPORTED;
    const size_t bytes = (size_t)(K / 32) * 2048 + 64;
    void* xa = nullptr;
    if (hipMallocAsync(&xa, bytes, st) != hipSuccess || !xa) {
        (void)hipGetLastError();
        return QMV_EUNSUPPORTED;
    }
    hipLaunchKernelGGL(k_xprep, dim3(16), dim3(XP_THREADS), 0, st, X, ldx, M, K, (uint8_t*)xa, (int*)nullptr, 0);
    int rc = check_launch("qmv activation pre-pass");
    if (rc == QMV_OK) {
        const long tiles = ((long)N + 15) / 16;
        const int ncu = num_cus();
        int tw = force_tw ? force_tw : (tiles >= 8L * ncu ? 2 : 1);
        const long groups = (tiles + tw - 1) / tw;
        const int P = K / 64;
        int S = 1;
        while (S < 8 && groups * S < 4L * ncu && (P + 2 * S - 1) / (2 * S) >= 4) S *= 2;
        if (force_S) S = force_S;
        MmPlan pl;
        pl.S = S;
        pl.seg = (P + S - 1) / S;
        pl.WR = 8 / S > 0 ? (S >= 8 ? 1 : 8 / S) : 1;
        if (pl.WR > 2 && groups < (long)ncu * pl.WR) pl.WR = 2;
        const long grid = (groups + pl.WR - 1) / pl.WR;
        if (tw == 2)
            hipLaunchKernelGGL((k_mm2<2>), dim3((unsigned)grid), dim3(64 * pl.S * pl.WR), 0, st, W, ldw, (const uint8_t*)xa, Y,
                               ldy, M, N, K, pl);
        else
            hipLaunchKernelGGL((k_mm2<1>), dim3((unsigned)grid), dim3(64 * pl.S * pl.WR), 0, st, W, ldw, (const uint8_t*)xa, Y,
                               ldy, M, N, K, pl);
        rc = check_launch("qmv mfma kernel");
    }
    if (hipFreeAsync(xa, st) != hipSuccess && rc == QMV_OK) rc = fail(QMV_EHIP, "qmv: hipFreeAsync failed");
    return rc;
}

// M = 2..16: activation pre-pass + k_mm3. Returns QMV_EUNSUPPORTED (nothing
// enqueued) when the shape is out of its range or scratch is unavailable.
int launch_mm3(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
               int force_S, int force_tw, hipStream_t st) {
    if (K > XP_KMAX) return QMV_EUNSUPPORTED;
    const int ncu = num_cus();
    const long tiles = ((long)N + 15) / 16;
    const int tw = force_tw ? force_tw : (tiles >= 2L * MM3_WAVES * 2 * ncu ? 2 : 1);
    const long groups = (tiles + (long)MM3_WAVES * tw - 1) / ((long)MM3_WAVES * tw);
    const int nchunks = (K + MM_KC - 1) / MM_KC;
    // Split-K across workgroups needs a device-wide release per workgroup,
    // which costs far more than it saves on this chip: one segment by default.
    int S = 1;
    if (force_S) S = force_S;
    S = S > nchunks ? nchunks : S;
    const int cps = (nchunks + S - 1) / S;
    S = (nchunks + cps - 1) / cps;
    if (groups > 0x7FFFFFFF || S > 65535) return QMV_EUNSUPPORTED;
    const size_t xa_bytes = (size_t)(K / 32) * 2048 + 64;
    const size_t part_bytes = S > 1 ? (size_t)S * groups * MM3_WAVES * tw * 64 * 16 : 0;
    const size_t arr_bytes = S > 1 ? (size_t)groups * 4 : 0;
    const size_t off_part = (xa_bytes + 255) & ~(size_t)255;
    const size_t off_arr = (off_part + part_bytes + 255) & ~(size_t)255;
    void* scratch = nullptr;
    if (hipMallocAsync(&scratch, off_arr + arr_bytes + 256, st) != hipSuccess || !scratch) {
        (void)hipGetLastError();
        return QMV_EUNSUPPORTED;
    }
    uint8_t* xa = (uint8_t*)scratch;
    float* part = (float*)(xa + off_part);
    int* arrive = (int*)(xa + off_arr);
    hipLaunchKernelGGL(k_xprep, dim3(16), dim3(XP_THREADS), 0, st, X, ldx, M, K, xa, arrive, (int)(arr_bytes / 4));
    int rc = check_launch("qmv activation pre-pass");
    if (rc == QMV_OK) {
        if (tw == 2)
            hipLaunchKernelGGL((k_mm3<2>), dim3((unsigned)groups, (unsigned)S), dim3(MM3_WAVES * 64), 2 * MM_CHUNK_BYTES, st, W,
                               ldw, (const uint8_t*)xa, Y, ldy, M, N, K, cps, part, arrive);
        else
            hipLaunchKernelGGL((k_mm3<1>), dim3((unsigned)groups, (unsigned)S), dim3(MM3_WAVES * 64), 2 * MM_CHUNK_BYTES, st, W,
                               ldw, (const uint8_t*)xa, Y, ldy, M, N, K, cps, part, arrive);
        rc = check_launch("qmv mfma kernel");
    }
    if (hipFreeAsync(scratch, st) != hipSuccess && rc == QMV_OK) rc = fail(QMV_EHIP, "qmv: hipFreeAsync failed");
    return rc;
}

template <int QT>
int launch_generic(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N,
                   int K, hipStream_t st) {
    const long grid = ((long)N + 3) / 4;
    if (grid > 0x7FFFFFFF) return fail(QMV_EINVAL, "N too large");
    if (M == 1)
        hipLaunchKernelGGL((k_generic<QT, 1>), dim3((unsigned)grid), dim3(256), 0, st, W, ldw, X, ldx, Y, ldy, M,
                           N, K);
    else
        hipLaunchKernelGGL((k_generic<QT, 16>), dim3((unsigned)grid), dim3(256), 0, st, W, ldw, X, ldx, Y, ldy, M,
                           N, K);
    return check_launch("qmv generic kernel");
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return na && nb && pa < pb + nb && pb < pa + na;
}

int dense(int qtype, const void* Wv, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
          void* stream) {
    const char* name = qtype == QMV_Q4_0 ? "qmv_q4_0" : "qmv_q8_0";
    const int bb = block_bytes(qtype);
    if (M < 0 || M > QMV_MAX_M) return fail(QMV_EUNSUPPORTED, "%s: M=%d outside 0..%d", name, M, QMV_MAX_M);
    if (N < 0) return fail(QMV_EINVAL, "%s: N=%d < 0", name, N);
    if (K < 0 || K % QK) return fail(QMV_EINVAL, "%s: K=%d is not a non-negative multiple of 32", name, K);
    if (M == 0 || N == 0) return QMV_OK;
    if (!Wv && K > 0) return fail(QMV_EINVAL, "%s: W is NULL", name);
    if (!X && K > 0) return fail(QMV_EINVAL, "%s: X is NULL", name);
    if (!Y) return fail(QMV_EINVAL, "%s: Y is NULL", name);
    const size_t row = (size_t)(K / QK) * bb;
    if (ldw < row) return fail(QMV_EINVAL, "%s: ldw_bytes=%zu < K/32*%d=%zu", name, ldw, bb, row);
    if (M > 1 && ldx < (size_t)K) return fail(QMV_EINVAL, "%s: ldx=%zu < K=%d", name, ldx, K);
    if (M > 1 && ldy < (size_t)N) return fail(QMV_EINVAL, "%s: ldy=%zu < N=%d", name, ldy, N);
    if (((uintptr_t)Wv & 1) || (ldw & 1)) return fail(QMV_EALIGN, "%s: W and ldw_bytes must be 2-byte aligned", name);
    if (((uintptr_t)X & 3) || ((uintptr_t)Y & 3)) return fail(QMV_EALIGN, "%s: X and Y must be 4-byte aligned", name);
    if (M == 1) ldx = (size_t)K, ldy = (size_t)N;
    if ((size_t)N > (SIZE_MAX - row) / (ldw ? ldw : 1)) return fail(QMV_EINVAL, "%s: N*ldw overflows", name);
    const size_t wbytes = K ? (size_t)(N - 1) * ldw + row : 0;
    const size_t xbytes = K ? ((size_t)(M - 1) * ldx + K) * 4 : 0;
    const size_t ybytes = ((size_t)(M - 1) * ldy + N) * 4;
    if (overlaps(Y, ybytes, Wv, wbytes) || overlaps(Y, ybytes, X, xbytes))
        return fail(QMV_EINVAL, "%s: Y overlaps W or X", name);

    hipStream_t st = (hipStream_t)stream;
    const uint8_t* W = (const uint8_t*)Wv;
    const bool fast_ok = M == 1 && K > 0 && K % 64 == 0 && K <= KMAX_FAST && ((uintptr_t)W & 3) == 0 &&
                         (ldw & 3) == 0 && ((uintptr_t)X & 3) == 0;
    if (fast_ok) {
        return qtype == QMV_Q4_0 ? launch_m1<QMV_Q4_0>(W, ldw, X, Y, N, K, st)
                                 : launch_m1<QMV_Q8_0>(W, ldw, X, Y, N, K, st);
    }
    const bool mm_ok = qtype == QMV_Q4_0 && M >= 2 && K > 0 && K % 64 == 0 && ((uintptr_t)W & 3) == 0 &&
                       (ldw & 3) == 0 && ((uintptr_t)X & 3) == 0;
    if (mm_ok) {
        const int rc = launch_mm3(W, ldw, X, ldx, Y, ldy, M, N, K, 0, 0, st);
        if (rc != QMV_EUNSUPPORTED) return rc;
        return launch_mm(W, ldw, X, ldx, Y, ldy, M, N, K, 0, 0, st);
    }
    return qtype == QMV_Q4_0 ? launch_generic<QMV_Q4_0>(W, ldw, X, ldx, Y, ldy, M, N, K, st)
                             : launch_generic<QMV_Q8_0>(W, ldw, X, ldx, Y, ldy, M, N, K, st);
}

template <int QT, int LPR, int RPT>
int launch_id_t(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
                int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err, int fast,
                hipStream_t st) {
    constexpr int WAVES = 4;
    constexpr int ROWS_PER_WG = (64 / LPR) * RPT * WAVES;
    const long tiles = ((long)N + ROWS_PER_WG - 1) / ROWS_PER_WG;
    if (tiles > 0x7FFFFFFF) return fail(QMV_EINVAL, "qmv_id: N too large");
    const size_t lds = fast ? xs_bytes(K) : 0;
    hipLaunchKernelGGL((k_id<QT, LPR, RPT, WAVES>), dim3((unsigned)tiles, (unsigned)n_pairs), dim3(WAVES * 64), lds,
                       st, W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, fast);
    return check_launch("qmv_id kernel");
}

template <int QT>
int launch_id(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
              int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err, int fast,
              hipStream_t st) {
    const int lpr = fast ? pick_lpr(K / 64) : 64;
#define QMV_ID_CASE(L) \
    if (lpr == L) return launch_id_t<QT, L, 1>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, fast, st);
    QMV_ID_CASE(64) QMV_ID_CASE(32) QMV_ID_CASE(16) QMV_ID_CASE(8) QMV_ID_CASE(4)
#undef QMV_ID_CASE
    return fail(QMV_EINVAL, "internal: no id kernel for lpr=%d", lpr);
}

}  // namespace

extern "C" {

int qmv_q4_0(const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
             void* stream) {
    return dense(QMV_Q4_0, W, ldw_bytes, X, ldx, Y, ldy, M, N, K, stream);
}

int qmv_q8_0(const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
             void* stream) {
    return dense(QMV_Q8_0, W, ldw_bytes, X, ldx, Y, ldy, M, N, K, stream);
}

int qmv_id(int qtype, const void* Wv, size_t expert_stride_bytes, size_t ldw_bytes, int n_experts, const float* X,
           size_t ldx, const uint32_t* ids, int n_tokens, int top_k, float* Y, size_t ldy, int N, int K,
           const float* expert_scale, int* err_flag, void* stream) {
    if (qtype != QMV_Q4_0 && qtype != QMV_Q8_0) return fail(QMV_EUNSUPPORTED, "qmv_id: qtype %d not supported", qtype);
    const int bb = block_bytes(qtype);
    if (n_experts <= 0) return fail(QMV_EINVAL, "qmv_id: n_experts=%d must be > 0", n_experts);
    if (top_k <= 0) return fail(QMV_EINVAL, "qmv_id: top_k=%d must be > 0", top_k);
    if (n_tokens < 0) return fail(QMV_EINVAL, "qmv_id: n_tokens=%d < 0", n_tokens);
    if (N < 0) return fail(QMV_EINVAL, "qmv_id: N=%d < 0", N);
    if (K < 0 || K % QK) return fail(QMV_EINVAL, "qmv_id: K=%d is not a non-negative multiple of 32", K);
    if (top_k > ID_MAX_LIST) return fail(QMV_EUNSUPPORTED, "qmv_id: top_k=%d exceeds %d", top_k, ID_MAX_LIST);
    if ((long)n_tokens * top_k > 0x7FFFFFFFL) return fail(QMV_EINVAL, "qmv_id: n_tokens*top_k overflows");
    if (n_tokens == 0 || N == 0) return QMV_OK;
    if (!Wv || !X || !ids || !Y) return fail(QMV_EINVAL, "qmv_id: NULL W, X, ids or Y");
    const size_t row = (size_t)(K / QK) * bb;
    if (ldw_bytes < row) return fail(QMV_EINVAL, "qmv_id: ldw_bytes=%zu < K/32*%d=%zu", ldw_bytes, bb, row);
    if ((size_t)N > SIZE_MAX / (ldw_bytes ? ldw_bytes : 1)) return fail(QMV_EINVAL, "qmv_id: N*ldw overflows");
    if (expert_stride_bytes < (size_t)N * ldw_bytes)
        return fail(QMV_EINVAL, "qmv_id: expert_stride_bytes=%zu < N*ldw_bytes=%zu", expert_stride_bytes,
                    (size_t)N * ldw_bytes);
    if (ldx < (size_t)K) return fail(QMV_EINVAL, "qmv_id: ldx=%zu < K=%d", ldx, K);
    if (ldy < (size_t)N) return fail(QMV_EINVAL, "qmv_id: ldy=%zu < N=%d", ldy, N);
    if (((uintptr_t)Wv & 1) || (ldw_bytes & 1) || (expert_stride_bytes & 1))
        return fail(QMV_EALIGN, "qmv_id: W, ldw_bytes and expert_stride_bytes must be 2-byte aligned");
    if (((uintptr_t)X & 3) || ((uintptr_t)Y & 3) || ((uintptr_t)ids & 3) || ((uintptr_t)expert_scale & 3) ||
        ((uintptr_t)err_flag & 3))
        return fail(QMV_EALIGN, "qmv_id: X, Y, ids, expert_scale and err_flag must be 4-byte aligned");
    const int n_pairs = n_tokens * top_k;
    const size_t ybytes = ((size_t)(n_pairs - 1) * ldy + N) * 4;
    const size_t wbytes = (size_t)(n_experts - 1) * expert_stride_bytes + (size_t)(N - 1) * ldw_bytes + row;
    const size_t xbytes = ((size_t)(n_tokens - 1) * ldx + K) * 4;
    if (overlaps(Y, ybytes, Wv, K ? wbytes : 0) || overlaps(Y, ybytes, X, K ? xbytes : 0) ||
        overlaps(Y, ybytes, ids, (size_t)n_pairs * 4) ||
        overlaps(Y, ybytes, expert_scale, expert_scale ? (size_t)n_experts * 4 : 0) ||
        overlaps(Y, ybytes, err_flag, err_flag ? 4 : 0))
        return fail(QMV_EINVAL, "qmv_id: Y overlaps another argument");

    hipStream_t st = (hipStream_t)stream;
    const uint8_t* W = (const uint8_t*)Wv;
    const int fast = K > 0 && K % 64 == 0 && K <= KMAX_FAST_ID && ((uintptr_t)W & 3) == 0 && (ldw_bytes & 3) == 0 &&
                     (expert_stride_bytes & 3) == 0;
    // A leader gathers at most ID_MAX_LIST pairs, so a call is split into
    // launches over whole tokens holding at most that many pairs each.
    const int tok_per_launch = ID_MAX_LIST / top_k;
    for (int t0 = 0; t0 < n_tokens; t0 += tok_per_launch) {
        const int nt = n_tokens - t0 < tok_per_launch ? n_tokens - t0 : tok_per_launch;
        const size_t p0 = (size_t)t0 * top_k;
        const float* Xs = X + (size_t)t0 * ldx;
        const uint32_t* is = ids + p0;
        float* Ys = Y + p0 * ldy;
        const int rc = qtype == QMV_Q4_0
                           ? launch_id<QMV_Q4_0>(W, expert_stride_bytes, ldw_bytes, n_experts, Xs, ldx, is, nt * top_k,
                                                 top_k, Ys, ldy, N, K, expert_scale, err_flag, fast, st)
                           : launch_id<QMV_Q8_0>(W, expert_stride_bytes, ldw_bytes, n_experts, Xs, ldx, is, nt * top_k,
                                                 top_k, Ys, ldy, N, K, expert_scale, err_flag, fast, st);
        if (rc) return rc;
    }
    return QMV_OK;
}

int qmv_batch(int qtype, const qmv_problem* problems, int n_problems, void* stream) {
    if (qtype != QMV_Q4_0 && qtype != QMV_Q8_0) return fail(QMV_EUNSUPPORTED, "qmv_batch: qtype %d not supported", qtype);
    if (n_problems < 0 || n_problems > QMV_MAX_BATCH)
        return fail(QMV_EINVAL, "qmv_batch: n_problems=%d outside 0..%d", n_problems, QMV_MAX_BATCH);
    if (n_problems == 0) return QMV_OK;
    if (!problems) return fail(QMV_EINVAL, "qmv_batch: problems is NULL");
    const int bb = block_bytes(qtype);
    size_t wb[QMV_MAX_BATCH], xb[QMV_MAX_BATCH], yb[QMV_MAX_BATCH];
    for (int i = 0; i < n_problems; ++i) {
        const qmv_problem& p = problems[i];
        if (p.N < 0) return fail(QMV_EINVAL, "qmv_batch: problem %d: N=%d < 0", i, p.N);
        if (p.K < 0 || p.K % QK) return fail(QMV_EINVAL, "qmv_batch: problem %d: K=%d is not a non-negative multiple of 32", i, p.K);
        const size_t row = (size_t)(p.K / QK) * bb;
        if (p.N > 0 && !p.y) return fail(QMV_EINVAL, "qmv_batch: problem %d: y is NULL", i);
        if (p.N > 0 && p.K > 0 && (!p.W || !p.x)) return fail(QMV_EINVAL, "qmv_batch: problem %d: W or x is NULL", i);
        if (p.ldw_bytes < row) return fail(QMV_EINVAL, "qmv_batch: problem %d: ldw_bytes=%zu < K/32*%d=%zu", i, p.ldw_bytes, bb, row);
        if (((uintptr_t)p.W & 1) || (p.ldw_bytes & 1)) return fail(QMV_EALIGN, "qmv_batch: problem %d: W and ldw_bytes must be 2-byte aligned", i);
        if (((uintptr_t)p.x & 3) || ((uintptr_t)p.y & 3)) return fail(QMV_EALIGN, "qmv_batch: problem %d: x and y must be 4-byte aligned", i);
        if (p.N > 0 && (size_t)p.N > (SIZE_MAX - row) / (p.ldw_bytes ? p.ldw_bytes : 1)) return fail(QMV_EINVAL, "qmv_batch: problem %d: N*ldw overflows", i);
        wb[i] = (p.N > 0 && p.K > 0) ? (size_t)(p.N - 1) * p.ldw_bytes + row : 0;
        xb[i] = (p.N > 0) ? (size_t)p.K * 4 : 0;
        yb[i] = (size_t)p.N * 4;
    }
    for (int i = 0; i < n_problems; ++i)
        for (int k = 0; k < n_problems; ++k) {
            if (overlaps(problems[i].y, yb[i], problems[k].W, wb[k]) || overlaps(problems[i].y, yb[i], problems[k].x, xb[k]) ||
                (k != i && overlaps(problems[i].y, yb[i], problems[k].y, yb[k])))
                return fail(QMV_EINVAL, "qmv_batch: output of problem %d overlaps an input or another output (problem %d)", i, k);
        }
    hipStream_t st = (hipStream_t)stream;
    M1Prob fast[QMV_MAX_BATCH];
    int nf = 0;
    for (int i = 0; i < n_problems; ++i) {
        const qmv_problem& p = problems[i];
        if (p.N == 0) continue;
        const uint8_t* W = (const uint8_t*)p.W;
        if (m1b_eligible(W, p.ldw_bytes, p.x, p.K)) {
            M1Prob& q = fast[nf++];
            q.W = W;
            q.x = p.x;
            q.y = p.y;
            q.ldw = p.ldw_bytes;
            q.N = p.N;
            q.K = p.K;
        } else {
            const int rc = qtype == QMV_Q4_0 ? launch_generic<QMV_Q4_0>(W, p.ldw_bytes, p.x, p.K, p.y, p.N, 1, p.N, p.K, st)
                                             : launch_generic<QMV_Q8_0>(W, p.ldw_bytes, p.x, p.K, p.y, p.N, 1, p.N, p.K, st);
            if (rc) return rc;
        }
    }
    if (nf == 0) return QMV_OK;
    return qtype == QMV_Q4_0 ? launch_m1b<QMV_Q4_0>(fast, nf, 0, 0, st) : launch_m1b<QMV_Q8_0>(fast, nf, 0, 0, st);
}

const char* qmv_last_error(void) { return g_err; }

#ifdef QMV_PROBE
// Tuning entries, built only into a separate probe library.
int qmv_probe_m1(int qtype, int lpr, int rpt, int waves, int wgs_per_cu, const void* W, size_t ldw, const float* X,
                 float* Y, int N, int K, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    const uint8_t* w = (const uint8_t*)W;
#define QMV_P(QT, L, R, WV)                            \
    if (qtype == QT && lpr == L && rpt == R && waves == WV) \
        return launch_m1_t<QT, L, R, WV>(w, ldw, X, Y, N, K, wgs_per_cu, st);
#define QMV_PW(QT, WV) QMV_P(QT, 64, 1, WV) QMV_P(QT, 64, 2, WV) QMV_P(QT, 32, 1, WV) QMV_P(QT, 32, 2, WV) \
    QMV_P(QT, 16, 1, WV) QMV_P(QT, 16, 2, WV)
    QMV_PW(QMV_Q4_0, 4) QMV_PW(QMV_Q4_0, 8) QMV_PW(QMV_Q4_0, 16)
    QMV_PW(QMV_Q8_0, 4) QMV_PW(QMV_Q8_0, 8) QMV_PW(QMV_Q8_0, 16)
#undef QMV_PW
#undef QMV_P
    return fail(QMV_EINVAL, "probe: no variant");
}

int qmv_probe_m1x(int qtype, int lpr, int rpt, int wr, int wgs_per_cu, const void* W, size_t ldw, const float* X,
                  float* Y, int N, int K, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    const uint8_t* w = (const uint8_t*)W;
    const float sc = qtype == QMV_Q4_0 ? 16.f : 1.f;
#define QMV_P(QT, L, R) \
    if (qtype == QT && lpr == L && rpt == R) return launch_m1x_t<QT, L, R>(w, ldw, X, Y, N, K, wr, wgs_per_cu, sc, st);
#define QMV_PQ(QT) QMV_P(QT, 64, 1) QMV_P(QT, 64, 2) QMV_P(QT, 32, 1) QMV_P(QT, 32, 2) QMV_P(QT, 16, 1) QMV_P(QT, 16, 2)
    QMV_PQ(QMV_Q4_0) QMV_PQ(QMV_Q8_0)
#undef QMV_PQ
#undef QMV_P
    return fail(QMV_EINVAL, "probe: no variant");
}

int qmv_probe_m1h(int target_wpc, int wgs_per_cu, int force_S, const void* W, size_t ldw, const float* X, float* Y,
                  int N, int K, void* stream) {
    return launch_m1h((const uint8_t*)W, ldw, X, Y, N, K, target_wpc, wgs_per_cu, force_S, (hipStream_t)stream);
}

int qmv_probe_m1o(int qtype, int maxi, int wpc, int n, const void* const* W, const size_t* ldw,
                   const float* const* X, float* const* Y, const int* N, const int* K, void* stream) {
    M1Prob p[MAXB];
    if (n < 1 || n > MAXB) return fail(QMV_EINVAL, "n");
    for (int i = 0; i < n; ++i) {
        p[i].W = (const uint8_t*)W[i];
        p[i].ldw = ldw[i];
        p[i].x = X[i];
        p[i].y = Y[i];
        p[i].N = N[i];
        p[i].K = K[i];
        if (!mo_eligible(p[i].W, p[i].ldw, p[i].x, p[i].K)) return fail(QMV_EINVAL, "not eligible");
    }
    return qtype == QMV_Q4_0 ? launch_m1o<QMV_Q4_0>(p, n, maxi, wpc, (hipStream_t)stream)
                             : launch_m1o<QMV_Q8_0>(p, n, maxi, wpc, (hipStream_t)stream);
}

int qmv_probe_m1q(int target_wpc, int wgs_per_cu, int force_S, int n, const void* const* W, const size_t* ldw,
                   const float* const* X, float* const* Y, const int* N, const int* K, void* stream) {
    M1Prob p[MAXB];
    if (n < 1 || n > MAXB) return fail(QMV_EINVAL, "n");
    for (int i = 0; i < n; ++i) {
        p[i].W = (const uint8_t*)W[i];
        p[i].ldw = ldw[i];
        p[i].x = X[i];
        p[i].y = Y[i];
        p[i].N = N[i];
        p[i].K = K[i];
        if (!mq_eligible(p[i].W, p[i].ldw, p[i].x, p[i].K)) return fail(QMV_EINVAL, "not eligible");
    }
    return launch_m1q(p, n, target_wpc, wgs_per_cu, force_S, (hipStream_t)stream);
}

int qmv_probe_m1b(int qtype, int waves, int wgs_per_cu, int n, const void* const* W, const size_t* ldw,
                  const float* const* X, float* const* Y, const int* N, const int* K, void* stream) {
    M1Prob pr[MAXB];
    for (int i = 0; i < n && i < MAXB; ++i) {
        pr[i].W = (const uint8_t*)W[i];
        pr[i].x = X[i];
        pr[i].y = Y[i];
        pr[i].ldw = ldw[i];
        pr[i].N = N[i];
        pr[i].K = K[i];
    }
    return qtype == QMV_Q4_0 ? launch_m1b<QMV_Q4_0>(pr, n, wgs_per_cu, waves, (hipStream_t)stream)
                             : launch_m1b<QMV_Q8_0>(pr, n, wgs_per_cu, waves, (hipStream_t)stream);
}

int qmv_probe_mm(int waves, int tw, const void* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M,
                 int N, int K, void* stream) {
    return launch_mm((const uint8_t*)W, ldw, X, ldx, Y, ldy, M, N, K, waves, tw, (hipStream_t)stream);
}

int qmv_probe_mm2(int S, int tw, const void* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M,
                  int N, int K, void* stream) {
    return launch_mm2((const uint8_t*)W, ldw, X, ldx, Y, ldy, M, N, K, S, tw, (hipStream_t)stream);
}

int qmv_probe_mm3(int S, int tw, const void* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M,
                  int N, int K, void* stream) {
    return launch_mm3((const uint8_t*)W, ldw, X, ldx, Y, ldy, M, N, K, S, tw, (hipStream_t)stream);
}
#endif

}  // extern "C"
