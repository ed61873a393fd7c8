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
//   * k_m1 / k_m1b   — M = 1 mat-vec (decode), one problem or a batch of up
//     to 16 (k_m1b picks the problem by workgroup index and runs the same
//     loop). Bandwidth-bound: every weight byte is read from HBM once. LPR
//     lanes cover one row, each lane streaming whole pairs of blocks (36 B
//     for Q4_0, 68 B for Q8_0) with dwordx4 loads, the next pair's loads in
//     flight while one is decoded; with LPR = 64 a wave reads a contiguous row.
//     The activation vector is staged once per workgroup into LDS (all 16-byte
//     loads issued before the stores, pairs padded to 68 floats so the lanes
//     of a read hit distinct banks). Q4_0 codes are decoded with
//     v_cvt_off_f32_i4 on (byte ^ 0x88), which yields (code - 8) / 16 exactly;
//     the 1/16 is undone once per output. A row's partial sums are reduced
//     across its LPR lanes with DPP moves.
//   * k_m1c          — the batched M = 1 call when all problems share x and K
//     (a layer's Q/K/V, its gate/up): their rows form one virtual matrix of
//     tiles that every workgroup strides through, so the work is even.
//   * k_mq (qmv_mq.hip) — Q4_0 and Q8_0 with M = 2..16 (and each 16-row
//     block of a prefill) on the matrix cores, one launch, no scratch memory.
//   * k_generic      — any qtype, 1..16 rows of X, any 2-byte alignment and
//     any K: one wave per weight row, one block per lane per step, 2-byte
//     loads. The fallback for shapes the fast kernels do not take.
//   * k_id           — expert-indexed product. One workgroup per (row tile,
//     (token, slot) pair). The workgroup of the first pair that selects an
//     expert ("leader") gathers every pair selecting the same expert and
//     streams that expert's rows once for all of them; other workgroups exit.
//
// All accumulation is fp32 in a fixed order (no atomics), so outputs are
// bitwise reproducible run to run.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>


#include "qmv.h"
#include "qmv_internal.h"

namespace qmvi {

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

}  // namespace qmvi

namespace {

using namespace qmvi;

constexpr int QK = 32;

__host__ __device__ constexpr int block_bytes(int qtype) { return qtype == QMV_Q4_0 ? 18 : 34; }

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// Signed int8 code in byte B of w, as float.
template <int B>
__device__ __forceinline__ float sbyte(uint32_t w) {
    return (float)(int8_t)(w >> (8 * B));
}


// Sum over one Q4_0 block whose 16 code bytes start at byte QB of the
// register window u[] (u = raw ^ 0x88888888, u4 = hi_nibbles(u)); xv = the block's
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
        u4[i] = hi_nibbles(u[i]);
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

// stage_x in two halves, so that other loads can be issued between them:
// stage_x_load issues this thread's 16-byte loads of x into v, stage_x_store
// writes them to the padded layout.
typedef float f32x4u_t __attribute__((ext_vector_type(4), aligned(4)));
template <int NT, int XCH>
__device__ __forceinline__ void stage_x_load(f32x4u_t (&v)[XCH], const float* __restrict__ x, int K) {
    const int nch = K >> 2;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int c = threadIdx.x + i * NT;
        if (c < nch) v[i] = *reinterpret_cast<const f32x4u_t*>(x + 4 * c);
    }
}
template <int NT, int XCH>
__device__ __forceinline__ void stage_x_store(float* xs, const f32x4u_t (&v)[XCH], int K) {
    const int nch = K >> 2;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int c = threadIdx.x + i * NT;
        if (c < nch)
            *reinterpret_cast<float4*>(xs + (c >> 4) * XS_PAIR + 4 * (c & 15)) = make_float4(v[i].x, v[i].y, v[i].z, v[i].w);
    }
}


// rows rows of x (row r at x + r * ldx, K values) into the padded layout, row
// r at xs + r * xstride; four 16-byte chunks in flight per thread (fewer
// registers than stage_x, for kernels that hold weight loads meanwhile).
template <int NT>
__device__ __forceinline__ void stage_rows(float* xs, size_t xstride, const float* __restrict__ x, size_t ldx,
                                           int rows, int K) {
    const int nch = K >> 2;
    const int total = rows * nch;
    for (int c0 = threadIdx.x; c0 < total; c0 += 4 * NT) {
        f32x4u_t a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + i * NT;
            if (c < total) {
                const int r = c / nch, cc = c - r * nch;
                a[i] = *reinterpret_cast<const f32x4u_t*>(x + (size_t)r * ldx + 4 * cc);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + i * NT;
            if (c < total) {
                const int r = c / nch, cc = c - r * nch;
                *reinterpret_cast<float4*>(xs + (size_t)r * xstride + (cc >> 4) * XS_PAIR + 4 * (cc & 15)) =
                    make_float4(a[i].x, a[i].y, a[i].z, a[i].w);
            }
        }
    }
}

// SiLU, z * sigmoid(z) = z / (1 + e^-z), in fp32. Below z = -88.7 e^-z
// overflows and the quotient is -0, the limit; NaN propagates.
__device__ __forceinline__ float silu_f(float z) { return z / (1.f + expf(-z)); }

// rows SwiGLU rows into the padded LDS layout, one after another (row r at
// xs + r * xstride): row r of the source holds 2K values at g + r * ldg, the
// gate half first, and its staged row is silu(gate) * up. NT threads, four
// 16-byte chunks of each half in flight per thread.
template <int NT>
__device__ __forceinline__ void stage_swiglu(float* xs, size_t xstride, const float* __restrict__ g, size_t ldg,
                                             int rows, int K) {
    typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
    const int nch = K >> 2;
    const int total = rows * nch;
    for (int c0 = threadIdx.x; c0 < total; c0 += 4 * NT) {
        f32x4u a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + i * NT;
            if (c < total) {
                const int r = c / nch, cc = c - r * nch;
                const float* src = g + (size_t)r * ldg + 4 * cc;
                a[i] = *reinterpret_cast<const f32x4u*>(src);
                b[i] = *reinterpret_cast<const f32x4u*>(src + K);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + i * NT;
            if (c < total) {
                const int r = c / nch, cc = c - r * nch;
                *reinterpret_cast<float4*>(xs + (size_t)r * xstride + (cc >> 4) * XS_PAIR + 4 * (cc & 15)) =
                    make_float4(silu_f(a[i].x) * b[i].x, silu_f(a[i].y) * b[i].y, silu_f(a[i].z) * b[i].z,
                                silu_f(a[i].w) * b[i].w);
            }
        }
    }
}

// nx activation rows gathered by pair into the padded layout, row i at
// xs + i * xstride: pair plist[i] uses row plist[i] / top_k of X (with SW the
// row holds 2K values and its SwiGLU is staged). The loads of all rows go out
// before any store (CH 16-byte chunks per thread at a time, half that with
// SW), so staging several rows costs about one memory latency, not one per
// row.
template <int NT, bool SW, int CH0 = 8>
__device__ __forceinline__ void stage_gather(float* xs, size_t xstride, const float* __restrict__ X, size_t ldx,
                                             const int* plist, int top_k, int nx, int K) {
    constexpr int CH = SW ? CH0 / 2 : CH0;
    const int nch = K >> 2;
    const int total = nx * nch;
    for (int c0 = threadIdx.x; c0 < total; c0 += CH * NT) {
        f32x4u_t a[CH], b[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = c0 + i * NT;
            if (c < total) {
                const int r = c / nch, cc = c - r * nch;
                const float* src = X + (size_t)(plist[r] / top_k) * ldx + 4 * cc;
                a[i] = *reinterpret_cast<const f32x4u_t*>(src);
                if constexpr (SW) b[i] = *reinterpret_cast<const f32x4u_t*>(src + K);
            }
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = c0 + i * NT;
            if (c < total) {
                const int r = c / nch, cc = c - r * nch;
                float4 v;
                if constexpr (SW)
                    v = make_float4(silu_f(a[i].x) * b[i].x, silu_f(a[i].y) * b[i].y, silu_f(a[i].z) * b[i].z,
                                    silu_f(a[i].w) * b[i].w);
                else
                    v = make_float4(a[i].x, a[i].y, a[i].z, a[i].w);
                *reinterpret_cast<float4*>(xs + (size_t)r * xstride + (cc >> 4) * XS_PAIR + 4 * (cc & 15)) = v;
            }
        }
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
// into LDS after the first loads are in flight (with SW, x holds 2K values and
// the staged row is their SwiGLU). Each row's sum is reduced over its lane
// group and written to y[row] * out_scale.
template <int QT, int LPR, int RPT, int WAVES, bool SW = false>
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
    // Two register buffers take turns: the next step's loads go into one
    // while the other is decoded, with no copy between them.
    uint32_t bufA[RPT][DW], bufB[RPT][DW];
    // This lane's rows of the tile being loaded: recomputed when a step
    // starts a tile (ldw < 2^32, so one 32 x 32 -> 64-bit multiply per row),
    // not every step.
    const uint8_t* irow[RPT];
    auto set_row = [&](long tl) {
        const long row0 = tl * ROWS + lrow;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const uint32_t rr = (uint32_t)(row0 + r < N ? row0 + r : N - 1);
            irow[r] = W + (uint64_t)rr * (uint32_t)ldw;
        }
    };
    auto issue = [&](int i, uint32_t (&b)[RPT][DW]) {
        int p = j + i * LPR;
        p = p < P ? p : P - 1;
#pragma unroll
        for (int r = 0; r < RPT; ++r) load_pair<DW>(irow[r] + (uint32_t)(p * PB), b[r]);
    };
    set_row(tile);
    if constexpr (SW) {
        issue(0, bufA);
        stage_swiglu<WAVES * 64>(xs, 0, x, 0, 1, K);
        __syncthreads();
    } else {
        // x loads first, then the first weight loads: waiting for x before
        // the LDS stores then leaves the weight loads in flight.
        constexpr int XCH = (KMAX_STAGE / 4 + WAVES * 64 - 1) / (WAVES * 64);
        f32x4u_t xv[XCH];
        stage_x_load<WAVES * 64, XCH>(xv, x, K);
        issue(0, bufA);
        stage_x_store<WAVES * 64, XCH>(xs, xv, K);
        wait_vmcnt<RPT * pair_loads<DW>()>();  // x loaded; only the weight loads remain
        lds_barrier();
    }
    float tot[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) tot[r] = 0.f;
    auto consume = [&](const uint32_t (&cb)[RPT][DW]) {
        // Lanes past the row end decode the clamped pair they loaded and add
        // zero: no branch around the decode, whose wait for this buffer's
        // loads must lie on every path (the next issue overwrites them).
        const int p = j + it * LPR;
        const bool in = p < P;
        const float4* xv = reinterpret_cast<const float4*>(xs + (in ? p : P - 1) * XS_PAIR);
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float d = T::dot(cb[r], xv);
            tot[r] += in ? d : 0.f;
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
    };
    // One step: issue the next step into `nb` and decode `cb`. Past the
    // last tile the loads are issued anyway (rows and pairs are clamped, the
    // data is never used), so that every step has the same shape and the
    // wait before each decode counts exactly the loads issued after it.
    auto step = [&](uint32_t (&cb)[RPT][DW], uint32_t (&nb)[RPT][DW]) {
        int it2 = it + 1;
        long tile2 = tile;
        if (it2 == IPT) {
            it2 = 0;
            tile2 += tile_stride;
            set_row(tile2);
        }
        issue(it2, nb);
#pragma unroll
        for (int r = 0; r < RPT; ++r) pin_regs<DW>(cb[r]);
        consume(cb);
        tile = tile2;
        it = it2;
    };
    // A counted loop with one exit: with an exit after each of the two
    // steps, the compiler joins the exits, and the joined path makes it wait
    // for the other buffer's loads before every issue.
    const long nsteps = ((ntiles - 1 - first_tile) / tile_stride + 1) * IPT;
    long s = 0;
    for (; s + 2 <= nsteps; s += 2) {
        step(bufA, bufB);
        step(bufB, bufA);
    }
    if (s < nsteps) step(bufA, bufB);
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
// Batched M = 1 kernel for problems that share one activation vector (the
// Q/K/V projections of a layer, or its FFN gate and up): the rows of all
// problems form one virtual matrix of tiles (problem p owns global tiles
// t0[p] .. t0[p+1]-1; a tile never spans two problems) and every workgroup
// takes tiles blockIdx.x, blockIdx.x + gridDim.x, ... of it, so the work is
// spread evenly whatever the problems' sizes, and x is staged once per
// workgroup. The loop is m1_stream's with one row per lane group, except
// that its two register buffers take turns instead of being copied.
// ---------------------------------------------------------------------------
// The problem table is sized for at most MAXP problems (1, 4 or 16): a
// kernel-argument block read before the first load is issued costs a small
// launch time in proportion to its size (a batch of one through the 16-entry
// table took 3.8 instead of 3.3 us on a 2 MB matrix).
template <int MAXP>
struct M1Cat {
    const uint8_t* W[MAXP];
    float* y[MAXP];
    size_t ldw[MAXP];
    int N[MAXP];
    long t0[MAXP + 1];
    const float* x;
    int K, n;
};

template <int QT, int LPR, int WAVES, int MAXP>
__global__ __launch_bounds__(WAVES * 64) void k_m1c(const M1Cat<MAXP> C) {
    extern __shared__ __align__(16) float xs[];
    using T = PairTraits<QT>;
    constexpr int DW = T::DW, PB = DW * 4;
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS = GROUPS * WAVES;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int K = C.K;
    const int P = K >> 6;
    const int IPT = (P + LPR - 1) / LPR;
    const long ntiles = C.t0[C.n];
    const long lrow = (long)(wave * GROUPS + g);
    const long stride = gridDim.x;
    long tile = blockIdx.x;
    if (tile >= ntiles) return;  // uniform over the workgroup
    // The parameters of the problem whose tile is being loaded (i*) and of
    // the one whose tile is being summed (s*) live in registers; the kernel
    // arguments are read again only when the loaded tile crosses into the
    // next problem.
    int ip = 0;
    if constexpr (MAXP > 1)
        while (ip + 1 < C.n && tile >= C.t0[ip + 1]) ++ip;
    const uint8_t* iW = C.W[ip];
    size_t ildw = C.ldw[ip];
    int iN = C.N[ip];
    long it0 = C.t0[ip], inext = C.t0[ip + 1];
    float* sy = C.y[ip];
    int sN = iN;
    long st0 = it0;
    int it = 0;
    // Two register buffers take turns: the next step's loads go into one
    // while the other is decoded, with no copy between them.
    uint32_t bufA[DW], bufB[DW];
    // This lane's row of the tile being loaded: recomputed when a step starts
    // a tile (ldw < 2^32, so one 32 x 32 -> 64-bit multiply), not every step.
    const uint8_t* irow = nullptr;
    auto set_row = [&](long tl) {
        const long row = (tl - it0) * ROWS + lrow;
        const uint32_t rr = (uint32_t)(row < iN ? row : iN - 1);
        irow = iW + (uint64_t)rr * (uint32_t)ildw;
    };
    auto issue = [&](int i, uint32_t (&b)[DW]) {
        int p = j + i * LPR;
        p = p < P ? p : P - 1;
        load_pair<DW>(irow + (uint32_t)(p * PB), b);
    };
    {
        constexpr int XCH = (KMAX_STAGE / 4 + WAVES * 64 - 1) / (WAVES * 64);
        f32x4u_t xv[XCH];
        stage_x_load<WAVES * 64, XCH>(xv, C.x, K);
        set_row(tile);
        issue(0, bufA);
        stage_x_store<WAVES * 64, XCH>(xs, xv, K);
        wait_vmcnt<pair_loads<DW>()>();  // x loaded; only the weight loads remain
        lds_barrier();
    }
    float tot = 0.f;
    // decode the current step from `cb`; write the row at the end of a tile
    auto consume = [&](const uint32_t (&cb)[DW]) {
        const int p = j + it * LPR;  // past the row end: decode the clamped pair, add zero (see m1_stream)
        const bool in = p < P;
        const float d = T::dot(cb, reinterpret_cast<const float4*>(xs + (in ? p : P - 1) * XS_PAIR));
        tot += in ? d : 0.f;
        if (it == IPT - 1) {
            const long row = (tile - st0) * ROWS + lrow;
            const float sum = lane_group_sum<LPR>(tot);
            if (j == LPR - 1 && row < sN) sy[row] = sum * T::OUT_SCALE;
            tot = 0.f;
        }
    };
    // One step: issue the next step into `nb` and decode `cb`.
    auto step = [&](uint32_t (&cb)[DW], uint32_t (&nb)[DW]) {
        int it2 = it + 1;
        long tile2 = tile;
        if (it2 == IPT) {
            it2 = 0;
            tile2 += stride;
            if constexpr (MAXP > 1) {
                if (tile2 >= inext && tile2 < ntiles) {
                    while (ip + 1 < C.n && tile2 >= C.t0[ip + 1]) ++ip;
                    iW = C.W[ip];
                    ildw = C.ldw[ip];
                    iN = C.N[ip];
                    it0 = C.t0[ip];
                    inext = C.t0[ip + 1];
                }
            }
        }
        // Past the last tile the loads are issued anyway (rows and pairs are
        // clamped, the data is never used), so that every step has the same
        // shape and the wait before each decode counts exactly the loads
        // issued after it.
        if (it2 == 0) set_row(tile2);
        issue(it2, nb);
        pin_regs<DW>(cb);
        consume(cb);
        if (it2 == 0) {  // the next step starts the tile just issued
            sy = C.y[ip];
            sN = iN;
            st0 = it0;
        }
        tile = tile2;
        it = it2;
    };
    // A counted loop with one exit: with an exit after each of the two
    // steps, the compiler joins the exits, and the joined path makes it wait
    // for the other buffer's loads before every issue.
    const long nsteps = ((ntiles - 1 - blockIdx.x) / stride + 1) * IPT;
    long s = 0;
    for (; s + 2 <= nsteps; s += 2) {
        step(bufA, bufB);
        step(bufB, bufA);
    }
    if (s < nsteps) step(bufA, bufB);
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
// With SW the rows of X hold 2K values and the activation is their SwiGLU,
// silu(X[k]) * X[K + k].
template <int QT, int MT, bool SW = false>
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
                auto xv = [&](int i) { return SW ? silu_f(xp[i]) * xp[K + i] : xp[i]; };
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s0 = fmaf(c[i], xv(i), s0);
                    s1 = fmaf(c[16 + i], xv(16 + i), s1);
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
// With SW the rows of X hold 2K values, gate then up, and the activation of
// token t is silu(gate) * up (the MoE down projection after SwiGLU).
// ---------------------------------------------------------------------------
// Decoded weights of one pair of blocks, for reuse against several
// activation vectors: w[0..31] block 0, w[32..63] block 1, as (code - 8) / 16
// (Q4_0) or code (Q8_0); d0, d1 the block scales.
template <int QT>
__device__ __forceinline__ void decode_pair(const uint32_t* r, float* w, float& d0, float& d1) {
    if constexpr (QT == QMV_Q4_0) {
        uint32_t u[9], u4[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) {
            u[i] = r[i] ^ 0x88888888u;
            u4[i] = hi_nibbles(u[i]);
        }
        unroll<0, 2>([&](auto R) {
            constexpr int QB = R ? 20 : 2;
            unroll<0, 16>([&](auto I) {
                constexpr int t = QB + I;
                w[32 * R + I] = nib<t % 4>(u[t / 4]);
                w[32 * R + 16 + I] = nib<t % 4>(u4[t / 4]);
            });
        });
        d0 = half_lo(r[0]);
        d1 = half_hi(r[4]);
    } else {
        unroll<0, 2>([&](auto R) {
            constexpr int QB = R ? 36 : 2;
            unroll<0, 32>([&](auto I) {
                constexpr int t = QB + I;
                w[32 * R + I] = sbyte<t % 4>(r[t / 4]);
            });
        });
        d0 = half_lo(r[0]);
        d1 = half_hi(r[8]);
    }
}

// Weights 16H .. 16H + 15 ((code - 8) / 16 for Q4_0, code for Q8_0) of
// block R (0 or 1) of a pair held in registers r, as decode_pair gives them.
template <int QT, int R, int H>
__device__ __forceinline__ void decode_half_w(const uint32_t* r, float* w) {
    if constexpr (QT == QMV_Q4_0) {
        constexpr int QB = R ? 20 : 2;  // the block's 16 code bytes: low nibbles 0..15, high 16..31
        uint32_t u[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            u[i] = r[QB / 4 + i] ^ 0x88888888u;
            if constexpr (H == 1) u[i] = hi_nibbles(u[i]);
        }
        unroll<0, 16>([&](auto I) {
            constexpr int t = QB % 4 + I;
            w[I] = nib<t % 4>(u[t / 4]);
        });
    } else {
        constexpr int QB = (R ? 36 : 2) + 16 * H;
        unroll<0, 16>([&](auto I) {
            constexpr int t = QB + I;
            w[I] = sbyte<t % 4>(r[t / 4]);
        });
    }
}

// m1_stream for nx <= MX activation vectors at once (the expert-indexed
// product when several (token, slot) pairs select one expert): each weight
// pair is loaded and decoded once and multiplied into every vector. The nx
// vectors x[i] (rows of X at xoff[i], or their SwiGLU with SW) are staged
// into LDS one after another; results go to y[i][row] * out_scale.
template <int QT, int LPR, int WAVES, int MX, bool SW = false>
__device__ __forceinline__ void m1_stream_mx(const uint8_t* __restrict__ W, size_t ldw, const float* __restrict__ X,
                                             const size_t* xoff, float* const* y, int nx, int N, int K,
                                             long first_tile, long tile_stride, float out_scale, float* xs) {
    using T = PairTraits<QT>;
    constexpr int DW = T::DW, PB = DW * 4;
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS = GROUPS * WAVES;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int P = K >> 6;
    const int IPT = (P + LPR - 1) / LPR;
    const long ntiles = ((long)N + ROWS - 1) / ROWS;
    const long lrow = (long)(wave * GROUPS + g);
    const size_t xstride = (size_t)P * XS_PAIR;  // floats per staged vector
    long tile = first_tile;
    if (tile >= ntiles) return;  // uniform over the workgroup
    int it = 0;
    uint32_t nxt[DW];
    auto issue = [&](long tl, int i) {
        long row = tl * ROWS + lrow;
        row = row < N ? row : N - 1;
        int p = j + i * LPR;
        p = p < P ? p : P - 1;
        load_pair<DW>(W + row * ldw + (size_t)p * PB, nxt);
    };
    issue(tile, 0);
#pragma unroll
    for (int i = 0; i < MX; ++i) {
        if (i < nx) {
            if constexpr (SW)
                stage_swiglu<WAVES * 64>(xs + i * xstride, 0, X + xoff[i], 0, 1, K);
            else
                stage_x<WAVES * 64, (KMAX_STAGE / 4 + WAVES * 64 - 1) / (WAVES * 64)>(xs + i * xstride, X + xoff[i], K);
        }
    }
    __syncthreads();
    float tot[MX];
#pragma unroll
    for (int i = 0; i < MX; ++i) tot[i] = 0.f;
    while (true) {
        uint32_t cur[DW];
#pragma unroll
        for (int d = 0; d < DW; ++d) cur[d] = nxt[d];
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
            float w[64], d0, d1;
            decode_pair<QT>(cur, w, d0, d1);
#pragma unroll
            for (int i = 0; i < MX; ++i) {
                if (i < nx) {
                    const float4* xv = reinterpret_cast<const float4*>(xs + i * xstride + p * XS_PAIR);
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const float4 a = xv[q], b = xv[8 + q];
                        s0 = fmaf(w[4 * q], a.x, s0);
                        s0 = fmaf(w[4 * q + 1], a.y, s0);
                        s0 = fmaf(w[4 * q + 2], a.z, s0);
                        s0 = fmaf(w[4 * q + 3], a.w, s0);
                        s1 = fmaf(w[32 + 4 * q], b.x, s1);
                        s1 = fmaf(w[32 + 4 * q + 1], b.y, s1);
                        s1 = fmaf(w[32 + 4 * q + 2], b.z, s1);
                        s1 = fmaf(w[32 + 4 * q + 3], b.w, s1);
                    }
                    tot[i] += fmaf(d1, s1, d0 * s0);
                }
            }
        }
        if (it == IPT - 1) {
            const long row = tile * ROWS + lrow;
#pragma unroll
            for (int i = 0; i < MX; ++i) {
                if (i < nx) {
                    const float sum = lane_group_sum<LPR>(tot[i]);
                    if (j == LPR - 1 && row < N) y[i][row] = sum * out_scale;
                }
                tot[i] = 0.f;
            }
        }
        if (!more) break;
        tile = tile2;
        it = it2;
    }
}

constexpr int ID_MAX_LIST = 1024;  // pairs one leader can serve in one pass
constexpr int ID_MX = 8;           // activation vectors streamed together

template <int QT, int LPR, int RPT, int WAVES, bool SW>
__global__ __launch_bounds__(WAVES * 64) void k_id(const uint8_t* __restrict__ W, size_t estride, size_t ldw,
                                                   int n_experts, const float* __restrict__ X, size_t ldx,
                                                   const uint32_t* __restrict__ ids, int n_pairs, int top_k,
                                                   float* __restrict__ Y, size_t ldy, int N, int K,
                                                   const float* __restrict__ escale, int* __restrict__ err_flag,
                                                   int fast, int mxcap) {
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

    if (fast) {
        const float sc = (escale ? escale[e] : 1.f) * PairTraits<QT>::OUT_SCALE;
        if (count == 1) {
            const int t = p / top_k;
            m1_stream<QT, LPR, RPT, WAVES, SW>(We, ldw, X + (size_t)t * ldx, Y + (size_t)p * ldy, N, K, blockIdx.x,
                                               gridDim.x, sc, xs);
            return;
        }
        // Several pairs: each weight pair is read once for up to mxcap of them.
        const int served = count < ID_MAX_LIST ? count : ID_MAX_LIST;
        for (int c0 = 0; c0 < served; c0 += mxcap) {
            const int nx = served - c0 < mxcap ? served - c0 : mxcap;
            size_t xoff[ID_MX];
            float* yp[ID_MX];
#pragma unroll
            for (int i = 0; i < ID_MX; ++i) {
                const int q = s_list[c0 + (i < nx ? i : nx - 1)];
                xoff[i] = (size_t)(q / top_k) * ldx;
                yp[i] = Y + (size_t)q * ldy;
            }
            if (c0 > 0) __syncthreads();  // the previous vectors' LDS reads are done
            m1_stream_mx<QT, LPR, WAVES, ID_MX, SW>(We, ldw, X, xoff, yp, nx, N, K, blockIdx.x, gridDim.x, sc, xs);
        }
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
            generic_row<QT, 16, SW>(We + n * ldw, X, xoff, M, K, lane, acc);
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
// Expert-indexed product grouped by expert, for calls with many pairs
// (batched decode, prefill). Every workgroup first groups the call's pairs by
// expert in LDS: the distinct experts u = 0 .. U-1 in order of first
// appearance and, for each, the pairs that select it. The rows of the
// distinct experts form one virtual matrix (virtual row v = u * N + n); each
// persistent workgroup takes an equal contiguous range of it, cut where the
// expert changes into segments. For a segment the workgroup stages the
// activation rows of its expert's pairs (mxcap at a time) and streams the
// segment's weight rows once, decoding each pair of blocks once and
// multiplying it into every staged row. So every selected expert is read once
// per call (once per mxcap of its pairs when more select it), with no
// workspace. A pair whose id is outside [0, n_experts) gets a NaN row and sets
// *err_flag. Per-pair results do not depend on how pairs are grouped, so the
// order of the atomics that fill the pair lists does not change any output.
// ---------------------------------------------------------------------------
constexpr int IDP_MX = 8;              // activation rows streamed together
// Rows per lane group. Two (the staged rows read once for both) measured
// slower on the MoE gate_up / down calls at 32 tokens (203 vs 163 us per
// pair of calls): fewer staged rows per pass and larger tiles.
constexpr int IDP_RPT = 1;

template <int QT, int LPR, int RPT, int WAVES, bool SW>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_idp(
    const uint8_t* __restrict__ W, size_t estride, size_t ldw, int n_experts, const float* __restrict__ X,
    size_t ldx, const uint32_t* __restrict__ ids, int n_pairs, int top_k, float* __restrict__ Y, size_t ldy, int N,
    int K, const float* __restrict__ escale, int* __restrict__ err_flag, int mxcap) {
    using T = PairTraits<QT>;
    constexpr int DW = T::DW, PB = DW * 4;
    constexpr int NT = WAVES * 64;
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS = GROUPS * RPT * WAVES;
    constexpr int MXR = IDP_MX / RPT;  // staged rows per pass (registers)
    __shared__ int s_map[IDP_MAX_EXPERTS];  // first pair of expert e, later its u
    __shared__ int s_uexp[IDP_MAX_PAIRS];   // expert of u
    __shared__ int s_ustart[IDP_MAX_PAIRS + 1];
    __shared__ int s_cnt[IDP_MAX_PAIRS];    // pairs of u, later the fill cursor
    __shared__ int s_plist[IDP_MAX_PAIRS];  // pairs grouped by u
    __shared__ int s_U;
    extern __shared__ __align__(16) float xs[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ---- group the pairs by expert ----
    // The tables are read by every lane at one address; readfirstlane tells
    // the compiler so, which keeps the values below in scalar registers and
    // the per-row tests `i < nx` scalar branches (as lane masks they cost a
    // few VALU instructions per staged row and half block).
    const int U = __builtin_amdgcn_readfirstlane(group_by_expert<NT>(
        ids, n_pairs, n_experts, s_map, s_uexp, s_ustart, s_cnt, s_plist, &s_U, Y, ldy, N, err_flag));
    auto ust = [&](int u) { return __builtin_amdgcn_readfirstlane(s_ustart[u]); };

    // ---- stream this workgroup's share of the virtual matrix ----
    const int g = lane / LPR, j = lane % LPR;
    const int P = K >> 6;
    const int IPT = (P + LPR - 1) / LPR;
    const size_t xstride = (size_t)P * XS_PAIR;
    // Work is split by cost, not rows: a row of expert u costs its pairs
    // plus 2 (the weight load and decode), so experts that many pairs select
    // spread over more workgroups. Row n of u sits at cost B(u) + n * c(u);
    // this workgroup takes the rows whose cost position is in [lo, hi).
    auto B = [&](int u) { return (long)N * (ust(u) + 2L * u); };
    const long C = B(U);
    const long lo = C * blockIdx.x / gridDim.x, hi = C * (blockIdx.x + 1) / gridDim.x;
    int u = 0;
    for (int span = 1 << 10; span > 0; span >>= 1)  // last u < U with B(u) <= lo
        if (u + span < U && B(u + span) <= lo) u += span;
    uint32_t bufA[RPT][DW], bufB[RPT][DW];
    bool staged = false;  // xs holds rows another segment may still be reading
    for (; u < U && B(u) < hi; ++u) {
        const int pbeg = ust(u), pend = ust(u + 1);
        const long cu = pend - pbeg + 2;
        const long a = lo - B(u), b = hi - B(u);
        const int n0 = a <= 0 ? 0 : (int)((a + cu - 1) / cu);
        const int n1 = (int)((b + cu - 1) / cu < N ? (b + cu - 1) / cu : N);
        if (n0 >= n1) continue;
        const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane(s_uexp[u]);
        const uint8_t* We = W + (size_t)e * estride;
        const float sc = (escale ? escale[e] : 1.f) * T::OUT_SCALE;
        const int ntl = (n1 - n0 + ROWS - 1) / ROWS;
        const int lrow = (wave * GROUPS + g) * RPT;  // this lane group's first row in a tile
        for (int c0 = pbeg; c0 < pend; c0 += mxcap) {
            const int nx = pend - c0 < mxcap ? pend - c0 : mxcap;
            int tile = 0, it = 0;
            auto issue = [&](int tl, int i, uint32_t (&b)[RPT][DW]) {
                int pp = j + i * LPR;
                pp = pp < P ? pp : P - 1;
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    int row = n0 + tl * ROWS + lrow + r;
                    row = row < n1 ? row : n1 - 1;
                    load_pair<DW>(We + (size_t)row * ldw + (size_t)pp * PB, b[r]);
                }
            };
            issue(0, 0, bufA);
            if (staged) lds_barrier();  // the previous rows' LDS reads are done
            // (fewer chunks in flight with two rows' weight loads pending)
            stage_gather<NT, SW, RPT == 1 ? 8 : 4>(xs, xstride, X, ldx, s_plist + c0, top_k, nx, K);
            wait_vmcnt<RPT * pair_loads<DW>()>();  // x loaded; only the weight loads remain
            lds_barrier();
            staged = true;
            float tot[RPT][MXR];
#pragma unroll
            for (int r = 0; r < RPT; ++r)
#pragma unroll
                for (int i = 0; i < MXR; ++i) tot[r][i] = 0.f;
            // decode each half block (16 weights) of the RPT pairs once and
            // multiply it into every staged row (x read once for the RPT
            // rows; 16 weights per row live at a time); the sums run over a
            // block's weights in order, as in the other kernels. Lanes past
            // the row end decode the clamped pair and add zero.
            auto consume = [&](const uint32_t (&cb)[RPT][DW]) {
                const int pp = j + it * LPR;
                const bool in = pp < P;
                const int pc = in ? pp : P - 1;
                float sb[2][RPT][MXR];  // per block
                unroll<0, 4>([&](auto RH) {
                    constexpr int R = RH / 2, H = RH % 2;
                    float w[RPT][16];
#pragma unroll
                    for (int r = 0; r < RPT; ++r) decode_half_w<QT, R, H>(cb[r], w[r]);
                    // a fresh scalar copy of nx per half block: the row tests
                    // stay scalar compares and branches, not lane masks
                    // hoisted out of the loop and rebuilt at every use
                    int nxh = nx;
                    asm volatile("" : "+s"(nxh));
#pragma unroll
                    for (int i = 0; i < MXR; ++i) {
                        if constexpr (H == 0) {
#pragma unroll
                            for (int r = 0; r < RPT; ++r) sb[R][r][i] = 0.f;
                        }
                        if (i < nxh) {
                            const float4* xv =
                                reinterpret_cast<const float4*>(xs + i * xstride + pc * XS_PAIR) + 8 * R + 4 * H;
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const float4 x4 = xv[q];
#pragma unroll
                                for (int r = 0; r < RPT; ++r) {
                                    sb[R][r][i] = fmaf(w[r][4 * q], x4.x, sb[R][r][i]);
                                    sb[R][r][i] = fmaf(w[r][4 * q + 1], x4.y, sb[R][r][i]);
                                    sb[R][r][i] = fmaf(w[r][4 * q + 2], x4.z, sb[R][r][i]);
                                    sb[R][r][i] = fmaf(w[r][4 * q + 3], x4.w, sb[R][r][i]);
                                }
                            }
                        }
                    }
                    // one half block at a time: hoisting the next decode
                    // above these products only holds more registers
                    __builtin_amdgcn_sched_barrier(0);
                });
                int nxt = nx;
                asm volatile("" : "+s"(nxt));
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    const float d0 = half_lo(cb[r][0]), d1 = QT == QMV_Q4_0 ? half_hi(cb[r][4]) : half_hi(cb[r][8]);
#pragma unroll
                    for (int i = 0; i < MXR; ++i) {
                        if (i < nxt) {
                            const float d = fmaf(d1, sb[1][r][i], d0 * sb[0][r][i]);
                            tot[r][i] += in ? d : 0.f;
                        }
                    }
                }
                if (it == IPT - 1) {
                    const int row0 = n0 + tile * ROWS + lrow;
#pragma unroll
                    for (int i = 0; i < MXR; ++i) {
                        if (i < nx) {
                            float* yr = Y + (size_t)__builtin_amdgcn_readfirstlane(s_plist[c0 + i]) * ldy;
#pragma unroll
                            for (int r = 0; r < RPT; ++r) {
                                const float sum = lane_group_sum<LPR>(tot[r][i]);
                                if (j == LPR - 1 && row0 + r < n1) yr[row0 + r] = sum * sc;
                            }
                        }
#pragma unroll
                        for (int r = 0; r < RPT; ++r) tot[r][i] = 0.f;
                    }
                }
            };
            // one step, the same shape every time (see m1_stream)
            auto step = [&](uint32_t (&cb)[RPT][DW], uint32_t (&nb)[RPT][DW]) {
                int it2 = it + 1, tile2 = tile;
                if (it2 == IPT) {
                    it2 = 0;
                    ++tile2;
                }
                issue(tile2, it2, nb);
#pragma unroll
                for (int r = 0; r < RPT; ++r) pin_regs<DW>(cb[r]);
                consume(cb);
                tile = tile2;
                it = it2;
            };
            const int nsteps = ntl * IPT;
            int st = 0;
            for (; st + 2 <= nsteps; st += 2) {
                step(bufA, bufB);
                step(bufB, bufA);
            }
            if (st < nsteps) step(bufA, bufB);
        }
    }
}

// ---------------------------------------------------------------------------
// Expert-indexed product for decode-sized calls (few pairs). The n_pairs x N
// output rows form one virtual matrix, virtual row v = p * N + n (row n of
// expert ids[p], output row p, activation row p / top_k), streamed by
// persistent workgroups with the M = 1 loop. Each workgroup stages every
// activation row of the call once (n_xrows of them; with SW their SwiGLU).
// Lane q of every wave holds ids[q] and that expert's scale, so a row's
// expert comes from a lane shuffle, not a memory load. Pairs that share an
// expert read it once each (the grouped kernel reads it once per call), so
// this is the kernel for a handful of pairs.
// ---------------------------------------------------------------------------
constexpr int IDV_MAX_PAIRS = 64;

template <int QT, int LPR, int WAVES, bool SW>
__global__ __launch_bounds__(WAVES * 64) void k_idv(const uint8_t* __restrict__ W, size_t estride, size_t ldw,
                                                    int n_experts, const float* __restrict__ X, size_t ldx,
                                                    const uint32_t* __restrict__ ids, int n_pairs, int top_k,
                                                    int n_xrows, float* __restrict__ Y, size_t ldy, int N, int K,
                                                    const float* __restrict__ escale, int* __restrict__ err_flag) {
    using T = PairTraits<QT>;
    constexpr int DW = T::DW, PB = DW * 4;
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS = GROUPS * WAVES;
    constexpr int NT = WAVES * 64;
    extern __shared__ __align__(16) float xs[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int P = K >> 6;
    const int IPT = (P + LPR - 1) / LPR;
    const int V = n_pairs * N;  // the host keeps this below 2^31
    const int ntiles = (V + ROWS - 1) / ROWS;
    const int lrow = wave * GROUPS + g;
    const size_t xstride = (size_t)P * XS_PAIR;

    int tile = blockIdx.x;
    if (tile >= ntiles) return;  // uniform over the workgroup
    const uint32_t idq = lane < n_pairs ? ids[lane] : 0u;

    // row of this lane group in tile tl: pair, row within the expert, expert
    auto rowinfo = [&](int tl, int& p, int& n, uint32_t& e) {
        int v = tl * ROWS + lrow;
        v = v < V ? v : V - 1;
        p = v / N;
        n = v - p * N;
        e = (uint32_t)__shfl((int)idq, p, 64);
    };
    auto wrow = [&](int n, uint32_t e) {
        return W + (size_t)(e < (uint32_t)n_experts ? e : 0u) * estride + (size_t)n * ldw;
    };
    // two register buffers in turn (see m1_stream)
    uint32_t bufA[DW], bufB[DW];
    auto issue = [&](const uint8_t* wr, int i, uint32_t (&b)[DW]) {
        int pp = j + i * LPR;
        pp = pp < P ? pp : P - 1;
        load_pair<DW>(wr + (size_t)pp * PB, b);
    };

    int p, n;
    uint32_t e;
    if constexpr (!SW) {
        if (n_xrows == 1) {
            // x loads first, then the first weight loads (see m1_stream)
            constexpr int XCH = (KMAX_STAGE / 4 + NT - 1) / NT;
            f32x4u_t xv[XCH];
            stage_x_load<NT, XCH>(xv, X, K);
            rowinfo(tile, p, n, e);
            issue(wrow(n, e), 0, bufA);
            stage_x_store<NT, XCH>(xs, xv, K);
        } else {
            rowinfo(tile, p, n, e);
            issue(wrow(n, e), 0, bufA);
            for (int r = 0; r < n_xrows; ++r)
                stage_x<NT, (KMAX_STAGE / 4 + NT - 1) / NT>(xs + r * xstride, X + (size_t)r * ldx, K);
        }
    } else {
        rowinfo(tile, p, n, e);
        issue(wrow(n, e), 0, bufA);
        stage_swiglu<NT>(xs, xstride, X, ldx, n_xrows, K);
    }
    wait_vmcnt<pair_loads<DW>()>();  // x loaded; only the weight loads remain
    // each pair's scale, needed first at the end of the first tile
    const float scq = lane < n_pairs && escale && idq < (uint32_t)n_experts ? escale[idq] : 1.f;
    lds_barrier();

    int it = 0;
    float tot = 0.f;
    auto consume = [&](const uint32_t (&cb)[DW]) {
        const int pp = j + it * LPR;  // past the row end: decode the clamped pair, add zero (see m1_stream)
        const bool in = pp < P;
        const float* xr = xs + (size_t)(p / top_k) * xstride + (in ? pp : P - 1) * XS_PAIR;
        const float d = T::dot(cb, reinterpret_cast<const float4*>(xr));
        tot += in ? d : 0.f;
        if (it == IPT - 1) {
            const float sc = __shfl(scq, p, 64) * T::OUT_SCALE;
            const float sum = lane_group_sum<LPR>(tot) * sc;
            const bool ok = e < (uint32_t)n_experts;
            const int v = tile * ROWS + lrow;
            if (j == LPR - 1 && v < V) {
                Y[(size_t)p * ldy + n] = ok ? sum : __builtin_nanf("");
                if (!ok && err_flag) *err_flag = 1;
            }
            tot = 0.f;
        }
    };
    // one step, the same shape every time (see m1_stream; rowinfo clamps
    // rows past the last tile)
    auto step = [&](uint32_t (&cb)[DW], uint32_t (&nb)[DW]) {
        int it2 = it + 1, tile2 = tile;
        int p2 = p, n2 = n;
        uint32_t e2 = e;
        if (it2 == IPT) {
            it2 = 0;
            tile2 += gridDim.x;
        }
        if (tile2 != tile) rowinfo(tile2, p2, n2, e2);
        issue(wrow(n2, e2), it2, nb);
        pin_regs<DW>(cb);
        consume(cb);
        tile = tile2;
        it = it2;
        p = p2;
        n = n2;
        e = e2;
    };
    const int nsteps = ((ntiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) * IPT;
    int s = 0;
    for (; s + 2 <= nsteps; s += 2) {
        step(bufA, bufB);
        step(bufB, bufA);
    }
    if (s < nsteps) step(bufA, bufB);
}

// The few-pairs kernel for rows of at most idv_deep(QT) steps per lane: all
// of a tile's weight loads are issued at once (one memory round trip per tile
// instead of one per step), and only the activation rows the tile uses are
// staged (x rows ta..tb of the tile's pairs go to LDS slots 0..tb-ta). The
// depth keeps the kernel within 128 VGPRs (4 waves per SIMD) without spills.
__host__ __device__ constexpr int idv_deep(int qt) { return qt == QMV_Q4_0 ? 4 : 2; }

template <int QT, int LPR, int WAVES, bool SW>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4))) void k_idv_deep(const uint8_t* __restrict__ W, size_t estride, size_t ldw,
                                                         int n_experts, const float* __restrict__ X, size_t ldx,
                                                         const uint32_t* __restrict__ ids, int n_pairs, int top_k,
                                                         float* __restrict__ Y, size_t ldy, int N, int K,
                                                         const float* __restrict__ escale, int* __restrict__ err_flag) {
    using T = PairTraits<QT>;
    constexpr int DW = T::DW, PB = DW * 4;
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS = GROUPS * WAVES;
    constexpr int NT = WAVES * 64;
    extern __shared__ __align__(16) float xs[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int P = K >> 6;
    constexpr int IDV_DEEP = idv_deep(QT);
    const int IPT = (P + LPR - 1) / LPR;  // at most IDV_DEEP (host)
    const int V = n_pairs * N;            // below 2^31 (host)
    const int ntiles = (V + ROWS - 1) / ROWS;
    const int lrow = wave * GROUPS + g;
    const size_t xstride = (size_t)P * XS_PAIR;

    int tile = blockIdx.x;
    if (tile >= ntiles) return;  // uniform over the workgroup
    const uint32_t idq = lane < n_pairs ? ids[lane] : 0u;
    float scq = 1.f;
    bool first = true;
    for (; tile < ntiles; tile += gridDim.x) {
        const int v0 = tile * ROWS;
        const int v1 = (v0 + ROWS < V ? v0 + ROWS : V) - 1;
        const int ta = (v0 / N) / top_k, tb = (v1 / N) / top_k;
        int v = v0 + lrow;
        v = v < V ? v : V - 1;
        const int p = v / N, n = v - p * N;
        const uint32_t e = (uint32_t)__shfl((int)idq, p, 64);
        const uint8_t* wr = W + (size_t)(e < (uint32_t)n_experts ? e : 0u) * estride + (size_t)n * ldw;
        uint32_t buf[IDV_DEEP][DW];
#pragma unroll
        for (int i = 0; i < IDV_DEEP; ++i) {
            if (i < IPT) {
                int pp = j + i * LPR;
                pp = pp < P ? pp : P - 1;
                load_pair<DW>(wr + (size_t)pp * PB, buf[i]);
            }
        }
        if (first) {  // each pair's scale, issued behind the first weight loads
            scq = lane < n_pairs && escale && idq < (uint32_t)n_experts ? escale[idq] : 1.f;
            first = false;
        }
        if constexpr (SW)
            stage_swiglu<NT>(xs, xstride, X + (size_t)ta * ldx, ldx, tb - ta + 1, K);
        else
            stage_rows<NT>(xs, xstride, X + (size_t)ta * ldx, ldx, tb - ta + 1, K);
        lds_barrier();
        const float* xr = xs + (size_t)(p / top_k - ta) * xstride;
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < IDV_DEEP; ++i) {
            const int pp = j + i * LPR;
            if (i < IPT && pp < P) tot += T::dot(buf[i], reinterpret_cast<const float4*>(xr + pp * XS_PAIR));
        }
        const float sc = __shfl(scq, p, 64) * T::OUT_SCALE;
        const float sum = lane_group_sum<LPR>(tot) * sc;
        const bool ok = e < (uint32_t)n_experts;
        if (j == LPR - 1 && v0 + lrow < V) {
            Y[(size_t)p * ldy + n] = ok ? sum : __builtin_nanf("");
            if (!ok && err_flag) *err_flag = 1;
        }
        lds_barrier();  // the next tile's staging overwrites xs
    }
}

// ---------------------------------------------------------------------------
// Routing-weighted sum over slots: out[t][n] = sum_s w[t*top_k + s] *
// Y[t*top_k + s][n], accumulated in slot order with one fma per slot.
// One thread per output element; the grid covers tokens x column tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_wsum(const float* __restrict__ Y, size_t ldy, const float* __restrict__ wts,
                                              int top_k, int N, long col_tiles, float* __restrict__ out, size_t ldo) {
    const long t = (long)blockIdx.x / col_tiles;
    const long n = ((long)blockIdx.x - t * col_tiles) * 256 + threadIdx.x;
    if (n >= N) return;
    const float* yp = Y + (size_t)t * top_k * ldy + n;
    const float* wp = wts + (size_t)t * top_k;
    float acc = 0.f;
    // slots in groups of 8: all loads of a group are issued before its fmas
    for (int s0 = 0; s0 < top_k; s0 += 8) {
        float yv[8], wv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int s = s0 + i < top_k ? s0 + i : top_k - 1;
            yv[i] = yp[(size_t)s * ldy];
            wv[i] = wp[s];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (s0 + i < top_k) acc = fmaf(wv[i], yv[i], acc);
    }
    out[(size_t)t * ldo + n] = acc;
}

// ---------------------------------------------------------------------------
// MoE down half of one token in one launch: SwiGLU of each slot's gate_up
// row, the down product of the slot's expert, and the weighted sum over
// slots. grid = (row tiles of R = 64 / LPR rows, tokens). Every slot's
// SwiGLU row is staged into LDS first; wave w then streams rows
// row0 .. row0 + R - 1 of the experts of slots w, w + WAVES, ... (LPR lanes
// per row, one step of register prefetch across slots) and puts each row's
// sum times expert_scale[e] into red[s][r]. Thread r < R then writes
// out[t][row0 + r] = sum_s w_s * red[s][r] in slot order. An id outside
// [0, n_experts) makes the token's rows NaN and sets *err_flag.
// Requires K % 64 == 0, top_k <= MD_MAX_TOPK, 4-byte aligned W, ldw and
// expert stride, and top_k staged rows within the LDS the host grants.
// ---------------------------------------------------------------------------
constexpr int MD_MAX_TOPK = 64;

template <int QT, int LPR, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_moe_down(const uint8_t* __restrict__ W, size_t estride, size_t ldw,
                                                         int n_experts, const float* __restrict__ G, size_t ldg,
                                                         const uint32_t* __restrict__ ids,
                                                         const float* __restrict__ wts, int top_k,
                                                         float* __restrict__ out, size_t ldo, int N, int K,
                                                         const float* __restrict__ escale, int* __restrict__ err_flag) {
    using T = PairTraits<QT>;
    constexpr int DW = T::DW, PB = DW * 4;
    constexpr int R = 64 / LPR;
    __shared__ float red[MD_MAX_TOPK][R];
    extern __shared__ __align__(16) float xs[];

    const long t = blockIdx.y;
    const long row0 = (long)blockIdx.x * R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int P = K >> 6;
    const int IPT = (P + LPR - 1) / LPR;
    const size_t xstride = (size_t)P * XS_PAIR;
    const uint32_t* tids = ids + t * top_k;
    long row = row0 + g;
    row = row < N ? row : N - 1;

    uint32_t nxt[DW];
    // This lane's row of slot sl's expert; an id out of range reads expert 0
    // (in bounds) and its result is replaced by NaN.
    auto base = [&](int sl) {
        uint32_t e = tids[sl];
        e = e < (uint32_t)n_experts ? e : 0u;
        return W + (size_t)e * estride + (size_t)row * ldw;
    };
    auto issue = [&](const uint8_t* b, int i) {
        int p = j + i * LPR;
        p = p < P ? p : P - 1;
        load_pair<DW>(b + (size_t)p * PB, nxt);
    };
    int s = wave, it = 0;
    const uint8_t* bn = W;
    if (s < top_k) {
        bn = base(s);
        issue(bn, 0);
    }
    stage_swiglu<WAVES * 64>(xs, xstride, G + (size_t)t * top_k * ldg, ldg, top_k, K);
    __syncthreads();
    float tot = 0.f;
    while (s < top_k) {  // uniform over the wave
        uint32_t cur[DW];
#pragma unroll
        for (int d = 0; d < DW; ++d) cur[d] = nxt[d];
        int it2 = it + 1, s2 = s;
        if (it2 == IPT) {
            it2 = 0;
            s2 += WAVES;
            if (s2 < top_k) bn = base(s2);
        }
        if (s2 < top_k) issue(bn, it2);
        pin_regs<DW>(cur);
        const int p = j + it * LPR;  // past the row end: decode the clamped pair, add zero (see m1_stream)
        const bool in = p < P;
        const float d = T::dot(cur, reinterpret_cast<const float4*>(xs + (size_t)s * xstride + (in ? p : P - 1) * XS_PAIR));
        tot += in ? d : 0.f;
        if (it == IPT - 1) {
            const uint32_t e = tids[s];
            const bool ok = e < (uint32_t)n_experts;
            const float sc = T::OUT_SCALE * (escale && ok ? escale[e] : 1.f);
            const float sum = lane_group_sum<LPR>(tot) * sc;
            if (j == LPR - 1) red[s][g] = ok ? sum : __builtin_nanf("");
            if (!ok && lane == 0 && err_flag) *err_flag = 1;
            tot = 0.f;
        }
        s = s2;
        it = it2;
    }
    __syncthreads();
    if (threadIdx.x < R) {
        const long r = row0 + threadIdx.x;
        if (r < N) {
            const float* wp = wts + t * top_k;
            float acc = 0.f;
            for (int k = 0; k < top_k; ++k) acc = fmaf(wp[k], red[k][threadIdx.x], acc);
            out[(size_t)t * ldo + r] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// Q6_K (GGML k-quant 6-bit super-blocks: 256 weights in 210 bytes).
// Super-block layout: ql[128] low 4 bits, qh[64] high 2 bits, 16 int8
// sub-block scales, binary16 d. Weight i: h = i / 128, r = i % 128,
// g = r / 32, l = r % 32; low bits = nibble (g / 2) of ql[64h + 32(g % 2) + l],
// high bits = bits 2g..2g+1 of qh[32h + l], q = low | high << 4, scale =
// scales[i / 16], w = d * scale * (q - 32).
//
// The kernel's unit is half a super-block (128 weights: 64 ql bytes, 32 qh
// bytes, 8 scales, and d): lanes take units as the Q4_0 kernels take pairs.
// Rows of an odd number of super-blocks are only 2-byte aligned; the loads
// use 2-byte aligned vector types, which gfx950 serves as unaligned global
// loads. sum (q - 32) x = sum q x - 32 sum x per 16-weight group, with the
// group sums of x computed once when x is staged.
// ---------------------------------------------------------------------------
constexpr int Q6_SB_BYTES = 210;
constexpr int Q6_UNIT_DW = 27;   // 16 ql + 8 qh + 2 scale dwords + d
constexpr int XS_Q6 = 132;       // LDS floats per staged unit (128 + 4 pad)
constexpr int KMAX_Q6 = 16384;   // largest K the Q6_K kernel stages

__host__ __device__ constexpr size_t q6_xs_bytes(int K) {
    return ((size_t)((K + 127) / 128) * XS_Q6 + (size_t)(K / 16)) * sizeof(float);
}

// Registers of unit h (0 or 1) of the super-block at sb.
__device__ __forceinline__ void load_q6_unit(const uint8_t* sb, int h, uint32_t* r) {
    typedef uint32_t u32x4a2 __attribute__((ext_vector_type(4), aligned(2)));
    typedef uint32_t u32x2a2 __attribute__((ext_vector_type(2), aligned(2)));
    const u32x4a2* ql = reinterpret_cast<const u32x4a2*>(sb + 64 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4a2 v = ql[i];
        r[4 * i] = v.x, r[4 * i + 1] = v.y, r[4 * i + 2] = v.z, r[4 * i + 3] = v.w;
    }
    const u32x4a2* qh = reinterpret_cast<const u32x4a2*>(sb + 128 + 32 * h);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const u32x4a2 v = qh[i];
        r[16 + 4 * i] = v.x, r[17 + 4 * i] = v.y, r[18 + 4 * i] = v.z, r[19 + 4 * i] = v.w;
    }
    const u32x2a2 sc = *reinterpret_cast<const u32x2a2*>(sb + 192 + 8 * h);
    r[24] = sc.x;
    r[25] = sc.y;
    // d is the high half of the dword ending the block (scales 14, 15 and
    // d): a 16-bit load would be zero-extended where the compiler chooses,
    // and that use makes it wait for all of a step's loads
    typedef uint32_t u32a2 __attribute__((aligned(2)));
    r[26] = *reinterpret_cast<const u32a2*>(sb + 206);
}

// Stage nx rows of x (row i at X + xoff[i]) for the Q6_K kernel: row i's
// unit u at xs + i * xstride + u * XS_Q6, and the sum of each 16-weight group
// j at gs + i * gstride + j. One thread per group of 16; loads are issued
// by stage_q6_load, and stored (with the sums) by stage_q6_store, so that
// weight loads can be issued between the two.
template <int NT, int GCH, int MX>
struct Q6Stage {
    f32x4u_t v[MX][GCH][4];
    __device__ __forceinline__ void load(const float* __restrict__ X, const size_t* xoff, int nx, int K) {
        const int ng = K >> 4;
#pragma unroll
        for (int i = 0; i < MX; ++i) {
            if (i < nx) {
#pragma unroll
                for (int c = 0; c < GCH; ++c) {
                    const int grp = threadIdx.x + c * NT;
                    if (grp < ng) {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            v[i][c][q] = *reinterpret_cast<const f32x4u_t*>(X + xoff[i] + 16 * grp + 4 * q);
                    }
                }
            }
        }
    }
    __device__ __forceinline__ void store(float* xs, size_t xstride, float* gs, size_t gstride, int nx, int K) {
        const int ng = K >> 4;
#pragma unroll
        for (int i = 0; i < MX; ++i) {
            if (i < nx) {
#pragma unroll
                for (int c = 0; c < GCH; ++c) {
                    const int grp = threadIdx.x + c * NT;
                    if (grp < ng) {
                        float* dst = xs + i * xstride + (grp >> 3) * XS_Q6 + 16 * (grp & 7);
                        float sum = 0.f;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x4u_t t = v[i][c][q];
                            *reinterpret_cast<float4*>(dst + 4 * q) = make_float4(t.x, t.y, t.z, t.w);
                            sum += (t.x + t.y) + (t.z + t.w);
                        }
                        gs[i * gstride + grp] = sum;
                    }
                }
            }
        }
    }
};

// tot[i] += dot of one unit (registers r) with staged row i (xs_i = its
// unit's 128 values, gs_i = its 8 group sums), for i < nx.
template <int MX>
__device__ __forceinline__ void q6_unit_dot(const uint32_t* r, const float* xs, size_t xstride, const float* gs,
                                            size_t gstride, int nx, float* tot) {
    const float d = half_hi(r[26]);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int is = 0; is < 2; ++is) {
            float acc[MX];
#pragma unroll
            for (int i = 0; i < MX; ++i) acc[i] = 0.f;
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                const int m = 4 * is + mm;
                const uint32_t lw = (g & 1) ? r[8 + m] : r[m];
                const uint32_t nib = (g < 2) ? (lw & 0x0F0F0F0Fu) : ((lw >> 4) & 0x0F0F0F0Fu);
                const uint32_t q = r[16 + m];
                const uint32_t hq = g == 0 ? (q << 4) : g == 1 ? (q << 2) : g == 2 ? q : (q >> 2);
                const uint32_t c = (hq & 0x30303030u) | nib;
                const float c0 = (float)(c & 0xFF), c1 = (float)((c >> 8) & 0xFF);
                const float c2 = (float)((c >> 16) & 0xFF), c3 = (float)(c >> 24);
#pragma unroll
                for (int i = 0; i < MX; ++i) {
                    if (i < nx) {
                        const float4 xv = *reinterpret_cast<const float4*>(xs + i * xstride + 32 * g + 4 * m);
                        acc[i] = fmaf(c0, xv.x, acc[i]);
                        acc[i] = fmaf(c1, xv.y, acc[i]);
                        acc[i] = fmaf(c2, xv.z, acc[i]);
                        acc[i] = fmaf(c3, xv.w, acc[i]);
                    }
                }
            }
            const int j = 2 * g + is;
            const float sc = (float)(int8_t)(r[24 + (j >> 2)] >> (8 * (j & 3)));
#pragma unroll
            for (int i = 0; i < MX; ++i)
                if (i < nx) tot[i] = fmaf(sc * d, fmaf(-32.f, gs[i * gstride + j], acc[i]), tot[i]);
        }
    }
}

// ---------------------------------------------------------------------------
// Q5_K (GGML k-quant 5-bit super-blocks: 256 weights in 176 bytes): d, dmin
// (binary16), 12 bytes of eight 6-bit sub-block scales and minimums, qh[32]
// (bit j of qh[l] = high bit of weight 32j + l), qs[128] (sub-blocks 2i, 2i+1
// in the low / high nibbles of qs[32i + l]). w = d * scale_j * q - dmin * min_j.
// The unit is again half a super-block: sub-blocks 4h .. 4h+3 (qs[64h ..
// 64h+63], all of qh, the 12 scale bytes, d and dmin).
// ---------------------------------------------------------------------------
constexpr int Q5_SB_BYTES = 176;
constexpr int Q5_UNIT_DW = 28;  // 16 qs + 8 qh + 3 scale dwords + d, dmin

__device__ __forceinline__ void load_q5_unit(const uint8_t* sb, int h, uint32_t* r) {
    typedef uint32_t u32x4a2 __attribute__((ext_vector_type(4), aligned(2)));
    typedef uint32_t u32x2a2 __attribute__((ext_vector_type(2), aligned(2)));
    typedef uint32_t u32a2 __attribute__((aligned(2)));
    const u32x4a2* qs = reinterpret_cast<const u32x4a2*>(sb + 48 + 64 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4a2 v = qs[i];
        r[4 * i] = v.x, r[4 * i + 1] = v.y, r[4 * i + 2] = v.z, r[4 * i + 3] = v.w;
    }
    const u32x4a2* qh = reinterpret_cast<const u32x4a2*>(sb + 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const u32x4a2 v = qh[i];
        r[16 + 4 * i] = v.x, r[17 + 4 * i] = v.y, r[18 + 4 * i] = v.z, r[19 + 4 * i] = v.w;
    }
    const u32x2a2 sc = *reinterpret_cast<const u32x2a2*>(sb + 4);
    r[24] = sc.x;
    r[25] = sc.y;
    r[26] = *reinterpret_cast<const u32a2*>(sb + 12);
    r[27] = *reinterpret_cast<const u32a2*>(sb);  // d (low half), dmin (high half)
}

// tot[i] += dot of Q5_K unit h (registers r) with staged row i.
template <int MX>
__device__ __forceinline__ void q5_unit_dot(const uint32_t* r, int h, const float* xs, size_t xstride,
                                            const float* gs, size_t gstride, int nx, float* tot) {
    const float d = half_lo(r[27]), dmin = half_hi(r[27]);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {  // sub-block j = 4h + jj
        // scale bytes jj, jj + 4, jj + 8 hold sub-blocks jj and jj + 4
        const uint32_t a = (r[24] >> (8 * jj)) & 0xFF, b = (r[25] >> (8 * jj)) & 0xFF;
        const uint32_t c = (r[26] >> (8 * jj)) & 0xFF;
        const uint32_t scj = h ? ((c & 15) | ((a >> 6) << 4)) : (a & 63);
        const uint32_t mnj = h ? ((c >> 4) | ((b >> 6) << 4)) : (b & 63);
        const int j = 4 * h + jj;
        float acc[MX];
#pragma unroll
        for (int i = 0; i < MX; ++i) acc[i] = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t w = r[8 * (jj >> 1) + m];
            const uint32_t nib = (jj & 1) ? ((w >> 4) & 0x0F0F0F0Fu) : (w & 0x0F0F0F0Fu);
            const uint32_t cq = nib | (((r[16 + m] >> j) & 0x01010101u) << 4);
            const float c0 = (float)(cq & 0xFF), c1 = (float)((cq >> 8) & 0xFF);
            const float c2 = (float)((cq >> 16) & 0xFF), c3 = (float)(cq >> 24);
#pragma unroll
            for (int i = 0; i < MX; ++i) {
                if (i < nx) {
                    const float4 xv = *reinterpret_cast<const float4*>(xs + i * xstride + 32 * jj + 4 * m);
                    acc[i] = fmaf(c0, xv.x, acc[i]);
                    acc[i] = fmaf(c1, xv.y, acc[i]);
                    acc[i] = fmaf(c2, xv.z, acc[i]);
                    acc[i] = fmaf(c3, xv.w, acc[i]);
                }
            }
        }
        const float dsc = d * (float)scj, dmn = dmin * (float)mnj;
#pragma unroll
        for (int i = 0; i < MX; ++i) {
            if (i < nx) {
                const float sx = gs[i * gstride + 2 * jj] + gs[i * gstride + 2 * jj + 1];
                tot[i] = fmaf(dsc, acc[i], fmaf(-dmn, sx, tot[i]));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// MLX affine 4-bit, groups of 32: a row's codes eight to a 32-bit word (code j
// in bits 4j), and one bf16 scale and one bf16 bias per group in arrays of
// their own; w = scale * q + bias. The unit is four groups (128 weights: 16
// code words, 4 scales, 4 biases); the last unit of a row whose K is not a
// multiple of 128 holds K % 128 weights and reads nothing past them.
// ---------------------------------------------------------------------------
constexpr int A4_UNIT_DW = 20;  // 16 code words + 2 scale dwords + 2 bias dwords

__device__ __forceinline__ void load_a4_unit(const uint8_t* wrow, const uint16_t* srow, const uint16_t* brow, int u,
                                             int K, uint32_t* r) {
    const int g0 = 4 * u, ng = K >> 5;  // groups of this unit: g0 .. g0 + 3, valid below ng
    const u32x4* wq = reinterpret_cast<const u32x4*>(wrow) + g0;
    uint16_t sv[4], bv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        u32x4 v = {0u, 0u, 0u, 0u};
        sv[g] = 0;
        bv[g] = 0;
        if (g0 + g < ng) {
            v = wq[g];
            sv[g] = srow[g0 + g];
            bv[g] = brow[g0 + g];
        }
        r[4 * g] = v.x, r[4 * g + 1] = v.y, r[4 * g + 2] = v.z, r[4 * g + 3] = v.w;
    }
    r[16] = sv[0] | (uint32_t)sv[1] << 16;
    r[17] = sv[2] | (uint32_t)sv[3] << 16;
    r[18] = bv[0] | (uint32_t)bv[1] << 16;
    r[19] = bv[2] | (uint32_t)bv[3] << 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// tot[i] += dot of affine unit u (registers r) with staged row i; groups at
// or past K (the tail of a row's last unit) contribute nothing.
template <int MX>
__device__ __forceinline__ void a4_unit_dot(const uint32_t* r, int u, int K, const float* xs, size_t xstride,
                                            const float* gs, size_t gstride, int nx, float* tot) {
    const int ng = K >> 5;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        if (4 * u + g >= ng) break;
        float acc[MX];
#pragma unroll
        for (int i = 0; i < MX; ++i) acc[i] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // weights 8w .. 8w+7 of the group
            const uint32_t q = r[4 * g + w];
            const uint32_t ev = q & 0x0F0F0F0Fu, od = (q >> 4) & 0x0F0F0F0Fu;  // even, odd weights
            const float c0 = (float)(ev & 0xFF), c2 = (float)((ev >> 8) & 0xFF);
            const float c4 = (float)((ev >> 16) & 0xFF), c6 = (float)(ev >> 24);
            const float c1 = (float)(od & 0xFF), c3 = (float)((od >> 8) & 0xFF);
            const float c5 = (float)((od >> 16) & 0xFF), c7 = (float)(od >> 24);
#pragma unroll
            for (int i = 0; i < MX; ++i) {
                if (i < nx) {
                    const float* xp = xs + i * xstride + 32 * g + 8 * w;
                    const float4 a = *reinterpret_cast<const float4*>(xp);
                    const float4 b = *reinterpret_cast<const float4*>(xp + 4);
                    acc[i] = fmaf(c0, a.x, acc[i]);
                    acc[i] = fmaf(c1, a.y, acc[i]);
                    acc[i] = fmaf(c2, a.z, acc[i]);
                    acc[i] = fmaf(c3, a.w, acc[i]);
                    acc[i] = fmaf(c4, b.x, acc[i]);
                    acc[i] = fmaf(c5, b.y, acc[i]);
                    acc[i] = fmaf(c6, b.z, acc[i]);
                    acc[i] = fmaf(c7, b.w, acc[i]);
                }
            }
        }
        const float sc = (g & 1) ? bf16_hi(r[16 + (g >> 1)]) : bf16_lo(r[16 + (g >> 1)]);
        const float bi = (g & 1) ? bf16_hi(r[18 + (g >> 1)]) : bf16_lo(r[18 + (g >> 1)]);
#pragma unroll
        for (int i = 0; i < MX; ++i)
            if (i < nx) tot[i] = fmaf(sc, acc[i], fmaf(bi, gs[i * gstride + 2 * g] + gs[i * gstride + 2 * g + 1], tot[i]));
    }
}

// The weight formats of the unit kernels below: units per row, the registers
// of unit u of a row (wrow: the row's bytes; srow, brow: its separate scales
// and biases, affine format only), and the unit's dot product.
struct FmtQ6K {
    static constexpr int DW = Q6_UNIT_DW, SB = Q6_SB_BYTES;
    __host__ __device__ static constexpr int units(int K) { return K >> 7; }
    __device__ static void load(const uint8_t* wrow, const uint16_t*, const uint16_t*, int u, int, uint32_t* r) {
        load_q6_unit(wrow + (size_t)(u >> 1) * Q6_SB_BYTES, u & 1, r);
    }
    template <int MX>
    __device__ static void dot(const uint32_t* r, int, int, const float* xs, size_t xstride, const float* gs,
                               size_t gstride, int nx, float* tot) {
        q6_unit_dot<MX>(r, xs, xstride, gs, gstride, nx, tot);
    }
};
struct FmtQ5K {
    static constexpr int DW = Q5_UNIT_DW, SB = Q5_SB_BYTES;
    __host__ __device__ static constexpr int units(int K) { return K >> 7; }
    __device__ static void load(const uint8_t* wrow, const uint16_t*, const uint16_t*, int u, int, uint32_t* r) {
        load_q5_unit(wrow + (size_t)(u >> 1) * Q5_SB_BYTES, u & 1, r);
    }
    template <int MX>
    __device__ static void dot(const uint32_t* r, int u, int, const float* xs, size_t xstride, const float* gs,
                               size_t gstride, int nx, float* tot) {
        q5_unit_dot<MX>(r, u & 1, xs, xstride, gs, gstride, nx, tot);
    }
};
struct FmtA4 {
    static constexpr int DW = A4_UNIT_DW;
    __host__ __device__ static constexpr int units(int K) { return (K + 127) >> 7; }
    __device__ static void load(const uint8_t* wrow, const uint16_t* srow, const uint16_t* brow, int u, int K,
                                uint32_t* r) {
        load_a4_unit(wrow, srow, brow, u, K, r);
    }
    template <int MX>
    __device__ static void dot(const uint32_t* r, int u, int K, const float* xs, size_t xstride, const float* gs,
                               size_t gstride, int nx, float* tot) {
        a4_unit_dot<MX>(r, u, K, xs, xstride, gs, gstride, nx, tot);
    }
};

// Persistent M <= MX kernel for a super-block format F: tiles of ROWS =
// (64 / LPR) * WAVES rows, tiles blockIdx.x, blockIdx.x + gridDim.x, ...;
// lane j of a row's LPR lanes takes units j, j + LPR, ... of the row, one
// step of register prefetch; row sums reduced over the lane group. Needs
// K % 256 == 0, 0 < K <= KMAX_Q6.
template <class F, int LPR, int WAVES, int MX>
__global__ __launch_bounds__(WAVES * 64) void k_q6k(const uint8_t* __restrict__ W, size_t ldw,
                                                     const float* __restrict__ X, size_t ldx, float* __restrict__ Y,
                                                     size_t ldy, int nx, int N, int K, const uint16_t* __restrict__ S,
                                                     const uint16_t* __restrict__ Bz, size_t lds) {
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS = GROUPS * WAVES;
    constexpr int NT = WAVES * 64;
    constexpr int GCH = (KMAX_Q6 / 16 + NT - 1) / NT;
    extern __shared__ __align__(16) float xs[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int U = F::units(K);
    const int IPT = (U + LPR - 1) / LPR;
    const long ntiles = ((long)N + ROWS - 1) / ROWS;
    const long lrow = (long)(wave * GROUPS + g);
    const size_t xstride = (size_t)U * XS_Q6;
    float* gs = xs + (size_t)nx * xstride;
    const size_t gstride = (size_t)(K >> 4);

    long tile = blockIdx.x;
    if (tile >= ntiles) return;  // uniform over the workgroup
    int it = 0;
    // two register buffers in turn (see m1_stream)
    uint32_t bufA[F::DW], bufB[F::DW];
    auto issue = [&](long tl, int i, uint32_t (&b)[F::DW]) {
        long row = tl * ROWS + lrow;
        row = row < N ? row : N - 1;
        int u = j + i * LPR;
        u = u < U ? u : U - 1;
        F::load(W + (size_t)row * ldw, S + (size_t)row * lds, Bz + (size_t)row * lds, u, K, b);
    };
    if constexpr (MX == 1) {
        // x loads first, then the first weight loads (see m1_stream)
        const size_t xo = 0;
        Q6Stage<NT, GCH, 1> stg;
        stg.load(X, &xo, 1, K);
        issue(tile, 0, bufA);
        stg.store(xs, 0, gs, 0, 1, K);
    } else {
        issue(tile, 0, bufA);
        for (int i = 0; i < nx; ++i) {
            const size_t xo = (size_t)i * ldx;
            Q6Stage<NT, GCH, 1> stg;
            stg.load(X, &xo, 1, K);
            stg.store(xs + i * xstride, 0, gs + i * gstride, 0, 1, K);
        }
    }
    lds_barrier();
    float tot[MX];
#pragma unroll
    for (int i = 0; i < MX; ++i) tot[i] = 0.f;
    auto consume = [&](const uint32_t (&cb)[F::DW]) {
        // past the row end: decode the clamped unit, add zero (see m1_stream)
        const int u0 = j + it * LPR;
        const bool in = u0 < U;
        const int u = in ? u0 : U - 1;
        float part[MX];
#pragma unroll
        for (int i = 0; i < MX; ++i) part[i] = 0.f;
        F::template dot<MX>(cb, u, K, xs + (size_t)u * XS_Q6, xstride, gs + 8 * u, gstride, nx, part);
#pragma unroll
        for (int i = 0; i < MX; ++i) tot[i] += in ? part[i] : 0.f;
        if (it == IPT - 1) {
            const long row = tile * ROWS + lrow;
#pragma unroll
            for (int i = 0; i < MX; ++i) {
                if (i < nx) {
                    const float sum = lane_group_sum<LPR>(tot[i]);
                    if (j == LPR - 1 && row < N) Y[(size_t)i * ldy + row] = sum;
                }
                tot[i] = 0.f;
            }
        }
    };
    // one step, the same shape every time (see m1_stream)
    auto step = [&](uint32_t (&cb)[F::DW], uint32_t (&nb)[F::DW]) {
        int it2 = it + 1;
        long tile2 = tile;
        if (it2 == IPT) {
            it2 = 0;
            tile2 += gridDim.x;
        }
        issue(tile2, it2, nb);
        pin_regs<F::DW>(cb);
        consume(cb);
        tile = tile2;
        it = it2;
    };
    const long nsteps = ((ntiles - 1 - (long)blockIdx.x) / gridDim.x + 1) * IPT;
    long s = 0;
    for (; s + 2 <= nsteps; s += 2) {
        step(bufA, bufB);
        step(bufB, bufA);
    }
    if (s < nsteps) step(bufA, bufB);
}

// Several M = 1 super-block products that share x and K in one launch
// (qmv_batch): the problems' rows are streamed as one virtual matrix of
// tiles, problem p owning tiles t0[p] .. t0[p + 1] - 1 (a tile never spans
// two problems), in k_q6k's loop. The loading tile's problem and the summing
// tile's output live in registers and change only at tile boundaries.
template <int MAXP>
struct Q6Cat {
    const uint8_t* W[MAXP];
    size_t ldw[MAXP];
    float* y[MAXP];
    int N[MAXP];
    long t0[MAXP + 1];
    const float* x;
    int K, n;
};

template <class F, int LPR, int WAVES, int MAXP>
__global__ __launch_bounds__(WAVES * 64) void k_q6kc(const Q6Cat<MAXP> C) {
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS = GROUPS * WAVES;
    constexpr int NT = WAVES * 64;
    constexpr int GCH = (KMAX_Q6 / 16 + NT - 1) / NT;
    extern __shared__ __align__(16) float xs[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int K = C.K;
    const int U = F::units(K);
    const int IPT = (U + LPR - 1) / LPR;
    const long ntiles = C.t0[C.n];
    const long lrow = (long)(wave * GROUPS + g);
    float* gs = xs + (size_t)U * XS_Q6;

    long tile = blockIdx.x;
    if (tile >= ntiles) return;  // uniform over the workgroup
    // The problem of a tile. Tile indices fit in 32 bits (the launch checks
    // it), and 32-bit compares stay scalar; as 64-bit compares they run on
    // the VALU, and the problem index, held in a vector register, then
    // makes every table read below a vector memory load on the step's path.
    auto prob = [&](long tl) {
        const int t = (int)tl;
        int ip = 0;
#pragma unroll
        for (int q = 1; q < MAXP; ++q) ip += (q < C.n && t >= (int)C.t0[q]) ? 1 : 0;
        return __builtin_amdgcn_readfirstlane(ip);
    };
    int ip = prob(tile);
    const uint8_t* iW = C.W[ip];
    size_t ildw = C.ldw[ip];
    int iN = C.N[ip];
    long it0 = C.t0[ip];
    float* sy = C.y[ip];
    int sN = iN;
    long st0 = it0;
    int it = 0;
    uint32_t bufA[F::DW], bufB[F::DW];
    auto issue = [&](long tl, int i, uint32_t (&b)[F::DW]) {
        long row = (tl - it0) * ROWS + lrow;
        row = row < iN ? row : iN - 1;
        int u = j + i * LPR;
        u = u < U ? u : U - 1;
        F::load(iW + (size_t)row * ildw, nullptr, nullptr, u, K, b);
    };
    {
        // x loads first, then the first weight loads (see m1_stream)
        const size_t xo = 0;
        Q6Stage<NT, GCH, 1> stg;
        stg.load(C.x, &xo, 1, K);
        issue(tile, 0, bufA);
        stg.store(xs, 0, gs, 0, 1, K);
    }
    lds_barrier();
    float tot = 0.f;
    auto consume = [&](const uint32_t (&cb)[F::DW]) {
        // past the row end: decode the clamped unit, add zero (see m1_stream)
        const int u0 = j + it * LPR;
        const bool in = u0 < U;
        const int u = in ? u0 : U - 1;
        float part[1] = {0.f};
        F::template dot<1>(cb, u, K, xs + (size_t)u * XS_Q6, 0, gs + 8 * u, 0, 1, part);
        tot += in ? part[0] : 0.f;
        if (it == IPT - 1) {
            const long row = (tile - st0) * ROWS + lrow;
            const float sum = lane_group_sum<LPR>(tot);
            if (j == LPR - 1 && row < sN) sy[row] = sum;
            tot = 0.f;
        }
    };
    // one step, the same shape every time (see m1_stream)
    auto step = [&](uint32_t (&cb)[F::DW], uint32_t (&nb)[F::DW]) {
        int it2 = it + 1;
        long tile2 = tile;
        if (it2 == IPT) {
            it2 = 0;
            tile2 += gridDim.x;
            if (tile2 < ntiles) {
                ip = prob(tile2);
                iW = C.W[ip];
                ildw = C.ldw[ip];
                iN = C.N[ip];
                it0 = C.t0[ip];
            }
        }
        issue(tile2, it2, nb);
        pin_regs<F::DW>(cb);
        consume(cb);
        if (it2 == 0) {  // the next step starts the tile just issued
            sy = C.y[ip];
            sN = iN;
            st0 = it0;
        }
        tile = tile2;
        it = it2;
    };
    const long nsteps = ((ntiles - 1 - (long)blockIdx.x) / gridDim.x + 1) * IPT;
    long s = 0;
    for (; s + 2 <= nsteps; s += 2) {
        step(bufA, bufB);
        step(bufB, bufA);
    }
    if (s < nsteps) step(bufA, bufB);
}

// Expert-indexed super-block (Q6_K, Q5_K) product: one workgroup per (tile of ROWS rows, pair
// p); expert ids[p]'s rows against activation row p / top_k. Pairs are not
// grouped by expert (each reads its expert's rows): the form for decode,
// where a token's experts are distinct. An id outside [0, n_experts) gives
// NaN rows and sets *err_flag.
template <class F, int LPR, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_id_q6(const uint8_t* __restrict__ W, size_t estride, size_t ldw,
                                                      int n_experts, const float* __restrict__ X, size_t ldx,
                                                      const uint32_t* __restrict__ ids, int top_k,
                                                      float* __restrict__ Y, size_t ldy, int N, int K,
                                                      const float* __restrict__ escale, int* __restrict__ err_flag,
                                                      const uint16_t* __restrict__ S, const uint16_t* __restrict__ Bz,
                                                      size_t s_estride, size_t lds) {
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS = GROUPS * WAVES;
    constexpr int NT = WAVES * 64;
    constexpr int GCH = (KMAX_Q6 / 16 + NT - 1) / NT;
    extern __shared__ __align__(16) float xs[];
    const int p = blockIdx.y;
    const uint32_t e = ids[p];
    const long row0 = (long)blockIdx.x * ROWS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int U = F::units(K);
    const int IPT = (U + LPR - 1) / LPR;
    if (e >= (uint32_t)n_experts) {  // uniform over the workgroup
        for (long n = row0 + tid; n < row0 + ROWS && n < N; n += NT) Y[(size_t)p * ldy + n] = __builtin_nanf("");
        if (tid == 0 && err_flag) *err_flag = 1;
        return;
    }
    const uint8_t* We = W + (size_t)e * estride;
    const long row = row0 + wave * GROUPS + g;
    const long rowc = row < N ? row : N - 1;
    float* gs = xs + (size_t)U * XS_Q6;
    uint32_t nxt[F::DW];
    auto issue = [&](int i) {
        int u = j + i * LPR;
        u = u < U ? u : U - 1;
        F::load(We + (size_t)rowc * ldw, S + (size_t)e * s_estride + (size_t)rowc * lds,
                Bz + (size_t)e * s_estride + (size_t)rowc * lds, u, K, nxt);
    };
    {
        // x loads first, then the first weight loads (see m1_stream)
        const size_t xo = (size_t)(p / top_k) * ldx;
        Q6Stage<NT, GCH, 1> stg;
        stg.load(X, &xo, 1, K);
        issue(0);
        stg.store(xs, 0, gs, 0, 1, K);
    }
    lds_barrier();
    float tot = 0.f;
    for (int it = 0; it < IPT; ++it) {
        uint32_t cur[F::DW];
#pragma unroll
        for (int d = 0; d < F::DW; ++d) cur[d] = nxt[d];
        if (it + 1 < IPT) issue(it + 1);
        const int u = j + it * LPR;
        if (u < U) F::template dot<1>(cur, u, K, xs + (size_t)u * XS_Q6, 0, gs + 8 * u, 0, 1, &tot);
    }
    const float sum = lane_group_sum<LPR>(tot) * (escale ? escale[e] : 1.f);
    if (j == LPR - 1 && row < N) Y[(size_t)p * ldy + row] = sum;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int KMAX_FAST = 15360;     // x staged in <= 64 KiB of LDS
constexpr int KMAX_FAST_ID = 14336;  // same, next to the id kernel's pair list

constexpr size_t LDS_PER_CU = 160 * 1024;  // gfx950


// Lanes per row: the largest power of two (<= 64) whose lane utilisation
// P / (LPR * ceil(P / LPR)) is within 5% of the best one, so long rows keep
// a full wave on one row and short rows still use every lane.
int pick_lpr(int P, int widest = 64) {
    const int cands[] = {64, 32, 16, 8, 4};
    double eff[5], best = 0;
    for (int i = 0; i < 5; ++i) {
        const int l = cands[i];
        eff[i] = l > widest ? 0. : (double)P / ((double)l * ((P + l - 1) / l));
        if (eff[i] > best) best = eff[i];
    }
    for (int i = 0; i < 5; ++i)
        if (eff[i] >= best * 0.95) return cands[i];
    return 4;
}

// Lanes per row of the dense M = 1 kernels: as pick_lpr, at most 32, so
// that rows of 64 pairs (K = 4096) take two steps per lane, which halves the
// per-row reductions and overlaps the decode of one step with the loads of
// the next (Q4_0 28672 x 4096: 14.0 vs 14.9 us; 4096 x 4096: 4.21 vs 4.38 us).
int pick_lpr_m1(int P) { return pick_lpr(P, 32); }

// Lanes per row for the Q6_K kernel (U units of 128 weights per row): the
// widest group whose lane utilisation U / (LPR * ceil(U / LPR)) is at least
// 0.85. A unit is twice a Q4_0 pair's work, so fewer sequential units per
// lane pays more than full lanes (K = 14336: 64 lanes at 0.875 beat 16 at 1.0
// by 1.4x).
int pick_lpr_q6(int U) {
    const int cands[] = {64, 32, 16, 8, 4};
    for (int l : cands)
        if ((double)U / ((double)l * ((U + l - 1) / l)) >= 0.85) return l;
    return 4;
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

// One M = 1 product: k_m1 with 8 waves, two workgroups per CU and the lane
// width of the row length. (As a batch of one through k_m1c the 2 MB call
// of 2048 x 2048 took 3.8 instead of 3.3 us: its larger kernel-argument
// block is read before anything else starts.)
template <int QT>
int launch_m1(const uint8_t* W, size_t ldw, const float* X, float* Y, int N, int K, hipStream_t st) {
    int lpr = pick_lpr_m1(K / 64);
    // Large matrices (at least two 32-row tiles per workgroup) with 1024 <=
    // K <= 8192: 16 lanes per row, so that a row's reduction and store come
    // once per several steps (Q4_0 65536 x 4096: 28.8 vs 31.1 us; 262144 x
    // 2816: 79.6 vs 83.2 us; Q8_0 262144 x 2816: 133.4 vs 137.0 us).
    if (N >= 32768 && K >= 1024 && K <= 8192) lpr = 16;
    switch (lpr) {
        case 32: return launch_m1_t<QT, 32, 1, 8>(W, ldw, X, Y, N, K, 2, st);
        case 16: return launch_m1_t<QT, 16, 1, 8>(W, ldw, X, Y, N, K, 2, st);
        case 8: return launch_m1_t<QT, 8, 1, 8>(W, ldw, X, Y, N, K, 2, st);
        default: return launch_m1_t<QT, 4, 1, 8>(W, ldw, X, Y, N, K, 2, st);
    }
}

// Plan for the x-stationary kernel: lanes per row and K segments.
bool m1b_eligible(const uint8_t* W, size_t ldw, const float* x, int K) {
    return K > 0 && K % 64 == 0 && K <= KMAX_FAST && ((uintptr_t)W & 3) == 0 && (ldw & 3) == 0 &&
           ldw <= 0xFFFFFFFFu && ((uintptr_t)x & 3) == 0;
}

// Launch the batched M = 1 kernel over n problems (n <= MAXB), all eligible.
// wgs_per_cu and waves are tuning knobs (0 = default).
template <int QT, int LPR, int MAXP>
int launch_m1c_t(const M1Cat<MAXP>& C, long tiles, int wgs_per_cu, hipStream_t st) {
    const size_t lds = xs_bytes(C.K);
    long per_cu = (long)(LDS_PER_CU / (lds ? lds : 1));
    per_cu = per_cu < 1 ? 1 : (per_cu < wgs_per_cu ? per_cu : wgs_per_cu);
    long grid = (long)num_cus() * per_cu;
    grid = grid < tiles ? grid : tiles;
    hipLaunchKernelGGL((k_m1c<QT, LPR, 8, MAXP>), dim3((unsigned)grid), dim3(512), lds, st, C);
    return check_launch("qmv shared-input batched m1 kernel");
}

// Problems that share x and K: one virtual matrix of 8-row tiles (k_m1c),
// with a problem table of MAXP >= n entries.
template <int QT, int MAXP>
int launch_m1c_n(const M1Prob* probs, int n, int wgs_per_cu, hipStream_t st) {
    M1Cat<MAXP> C;
    C.x = probs[0].x;
    C.K = probs[0].K;
    C.n = n;
    const int lpr = pick_lpr_m1(C.K / 64);
    const long rows = (long)(64 / lpr) * 8;
    C.t0[0] = 0;
    for (int i = 0; i < n; ++i) {
        C.W[i] = probs[i].W;
        C.y[i] = probs[i].y;
        C.ldw[i] = probs[i].ldw;
        C.N[i] = probs[i].N;
        C.t0[i + 1] = C.t0[i] + ((long)probs[i].N + rows - 1) / rows;
    }
    const long tiles = C.t0[n];
    if (tiles > 0x7FFFFFFF) return fail(QMV_EINVAL, "N too large");
    switch (lpr) {
        case 32: return launch_m1c_t<QT, 32, MAXP>(C, tiles, wgs_per_cu, st);
        case 16: return launch_m1c_t<QT, 16, MAXP>(C, tiles, wgs_per_cu, st);
        case 8: return launch_m1c_t<QT, 8, MAXP>(C, tiles, wgs_per_cu, st);
        default: return launch_m1c_t<QT, 4, MAXP>(C, tiles, wgs_per_cu, st);
    }
}

template <int QT>
int launch_m1c(const M1Prob* probs, int n, int wgs_per_cu, hipStream_t st) {
    if (n <= 1) return launch_m1c_n<QT, 1>(probs, n, wgs_per_cu, st);
    if (n <= 4) return launch_m1c_n<QT, 4>(probs, n, wgs_per_cu, st);
    return launch_m1c_n<QT, MAXB>(probs, n, wgs_per_cu, st);
}

template <int QT>
int launch_m1b(const M1Prob* probs, int n, int wgs_per_cu, int waves, hipStream_t st) {
    if (waves == 0) waves = 8;
    if (wgs_per_cu == 0) wgs_per_cu = 2;
    bool shared = waves == 8;
    for (int i = 1; i < n; ++i) shared = shared && probs[i].x == probs[0].x && probs[i].K == probs[0].K;
    if (shared) return launch_m1c<QT>(probs, n, wgs_per_cu, st);
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

// The dense product (qmv_q4_0 / qmv_q8_0 / qmv_ws): validation, then the
// kernel for the shape. ws: an optional caller workspace for M >= 2
// (ws_bytes of it), overlap-checked like the outputs.
int dense(int qtype, const void* Wv, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
          void* stream, void* ws = nullptr, size_t ws_bytes = 0, const char* name = nullptr) {
    if (!name) name = qtype == QMV_Q4_0 ? "qmv_q4_0" : "qmv_q8_0";
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
    if (ws && (((uintptr_t)ws & 255) || overlaps(ws, ws_bytes, Y, ybytes) || overlaps(ws, ws_bytes, Wv, wbytes) ||
               overlaps(ws, ws_bytes, X, xbytes)))
        return fail(QMV_EINVAL, "%s: the workspace must be 256-byte aligned and not overlap W, X or Y", name);

    hipStream_t st = (hipStream_t)stream;
    const uint8_t* W = (const uint8_t*)Wv;
    const bool fast_ok = M == 1 && K > 0 && K % 64 == 0 && K <= KMAX_FAST && ((uintptr_t)W & 3) == 0 &&
                         (ldw & 3) == 0 && ldw <= 0xFFFFFFFFu && ((uintptr_t)X & 3) == 0;
    if (fast_ok) {
        return qtype == QMV_Q4_0 ? launch_m1<QMV_Q4_0>(W, ldw, X, Y, N, K, st)
                                 : launch_m1<QMV_Q8_0>(W, ldw, X, Y, N, K, st);
    }
    const bool mq_ok = M >= 2 && K > 0 && K % 64 == 0 && ((uintptr_t)W & 3) == 0 && (ldw & 3) == 0;
    if (mq_ok) return launch_mq(qtype, W, ldw, X, ldx, Y, ldy, M, N, K, ws, ws ? ws_bytes : 0, st);
    return qtype == QMV_Q4_0 ? launch_generic<QMV_Q4_0>(W, ldw, X, ldx, Y, ldy, M, N, K, st)
                             : launch_generic<QMV_Q8_0>(W, ldw, X, ldx, Y, ldy, M, N, K, st);
}

template <int QT, int LPR, int RPT, bool SW, int WAVES = 4>
int launch_id_t(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
                int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err, int fast,
                hipStream_t st) {
    constexpr int ROWS_PER_WG = (64 / LPR) * RPT * WAVES;
    const long tiles = ((long)N + ROWS_PER_WG - 1) / ROWS_PER_WG;
    if (tiles > 0x7FFFFFFF) return fail(QMV_EINVAL, "qmv_id: N too large");
    // LDS for up to ID_MX staged vectors, within 64 KiB
    int mxcap = 1;
    if (fast) {
        const size_t one = xs_bytes(K);
        mxcap = (int)(65536 / (one ? one : 1));
        mxcap = mxcap < 1 ? 1 : (mxcap > ID_MX ? ID_MX : mxcap);
    }
    const size_t lds = fast ? (size_t)mxcap * xs_bytes(K) : 0;
    hipLaunchKernelGGL((k_id<QT, LPR, RPT, WAVES, SW>), dim3((unsigned)tiles, (unsigned)n_pairs), dim3(WAVES * 64), lds,
                       st, W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, fast, mxcap);
    return check_launch("qmv_id kernel");
}

// The grouped kernel k_idp: 8 waves, two workgroups per CU when two staged
// rows fit in the LDS that leaves (else one), as many staged rows per pass
// as fit, at most IDP_MX.
template <int QT, int LPR, int RPT, bool SW>
int launch_idp_t(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
                 int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err,
                 hipStream_t st) {
    constexpr int WAVES = 8;
    constexpr size_t STATIC_LDS = (size_t)(IDP_MAX_EXPERTS + 4 * IDP_MAX_PAIRS + 2) * sizeof(int);
    const size_t one = xs_bytes(K);
    int per_cu = 2;
    long mx = (long)((LDS_PER_CU / 2 - STATIC_LDS) / one);
    if (mx < 2) {
        per_cu = 1;
        mx = (long)((LDS_PER_CU - STATIC_LDS) / one);
    }
    mx = mx > IDP_MX / RPT ? IDP_MX / RPT : mx;
    if (mx < 1) return fail(QMV_EINVAL, "internal: K=%d too large for the grouped id kernel", K);
    // at most min(n_pairs, E) distinct experts of N rows each
    const long umax = n_pairs < E ? n_pairs : E;
    const long rows = (64 / LPR) * RPT * WAVES;
    const long tiles = (umax * N + rows - 1) / rows;
    long grid = (long)num_cus() * per_cu;
    grid = grid < tiles ? grid : tiles;
    grid = grid < 1 ? 1 : grid;
    hipLaunchKernelGGL((k_idp<QT, LPR, RPT, WAVES, SW>), dim3((unsigned)grid), dim3(WAVES * 64), (size_t)mx * one, st, W,
                       es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, (int)mx);
    return check_launch("qmv_id grouped kernel");
}

template <int QT, bool SW>
int launch_idp(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
               int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err,
               hipStream_t st) {
    const int lpr = pick_lpr(K / 64);
#define QMV_IDP_CASE(L) \
    if (lpr == L) return launch_idp_t<QT, L, IDP_RPT, SW>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, st);
    QMV_IDP_CASE(64) QMV_IDP_CASE(32) QMV_IDP_CASE(16) QMV_IDP_CASE(8) QMV_IDP_CASE(4)
#undef QMV_IDP_CASE
    return fail(QMV_EINVAL, "internal: no grouped id kernel for lpr=%d", lpr);
}

template <int QT, int LPR, bool SW>
int launch_idv_t(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
                 int n_pairs, int top_k, int n_xrows, float* Y, size_t ldy, int N, int K, const float* sc, int* err,
                 int wgs_per_cu, int deep, hipStream_t st) {
    constexpr int WAVES = 8;
    constexpr int ROWS = (64 / LPR) * WAVES;
    const long tiles = ((long)n_pairs * N + ROWS - 1) / ROWS;
    long nwg = (long)num_cus() * (wgs_per_cu > 0 ? wgs_per_cu : 2);
    nwg = nwg < tiles ? nwg : tiles;
    const int ipt = (K / 64 + LPR - 1) / LPR;
    // All loads at once pays when tiles restage few of several x rows; with
    // one x row, staging it once per workgroup and streaming is faster.
    if (deep < 0) deep = ipt <= idv_deep(QT) && n_xrows > 1;
    if (deep && ipt <= idv_deep(QT)) {
        // x rows one tile can touch: the pairs of ROWS consecutive rows
        long xr = (long)(ROWS - 1) / N + 2;
        xr = xr < n_xrows ? xr : n_xrows;
        hipLaunchKernelGGL((k_idv_deep<QT, LPR, WAVES, SW>), dim3((unsigned)nwg), dim3(WAVES * 64),
                           (size_t)xr * xs_bytes(K), st, W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc,
                           err);
    } else {
        hipLaunchKernelGGL((k_idv<QT, LPR, WAVES, SW>), dim3((unsigned)nwg), dim3(WAVES * 64),
                           (size_t)n_xrows * xs_bytes(K), st, W, es, ldw, E, X, ldx, ids, n_pairs, top_k, n_xrows, Y,
                           ldy, N, K, sc, err);
    }
    return check_launch("qmv_id kernel (few pairs)");
}

// Lanes per row for the few-pairs kernel: the efficient choice for the row
// length, widened while the call has fewer than two tiles per compute unit
// (these calls are latency-bound: more, shorter lane chains). Measured on the
// MoE decode calls (gate_up 8 x 1408 x 2816: 4 -> 16 lanes, 11.6 -> 8.3 us;
// SwiGLU-fed down 8 x 2816 x 704: 4 -> 16 lanes, all loads at once).
int pick_lpr_idv(int P, long rows) {
    int lpr = pick_lpr(P);
    while (lpr < 64 && (rows + (64 / lpr) * 8 - 1) / ((64 / lpr) * 8) < 2L * num_cus()) lpr *= 2;
    return lpr;
}

// Launch plan of the few-pairs kernel: lanes per row, whether all of a
// tile's loads go out at once, and the LDS for the staged x rows. Lanes are
// widened until the staged rows fit in 64 KiB (wider rows take fewer steps,
// which allows the per-tile staging of the all-at-once variant); false when
// nothing fits (the grouped kernel then runs).
struct IdvPlan {
    int lpr, deep;
    size_t lds;
};
bool plan_idv(int qt, int K, int n_pairs, int N, int n_xrows, IdvPlan& pl) {
    const int P = K / 64;
    for (int lpr = pick_lpr_idv(P, (long)n_pairs * N);; lpr *= 2) {
        const int ipt = (P + lpr - 1) / lpr;
        const int deep = ipt <= idv_deep(qt) && n_xrows > 1;
        const long rows_per_tile = (64 / lpr) * 8;
        long xr = deep ? (rows_per_tile - 1) / N + 2 : n_xrows;
        xr = xr < n_xrows ? xr : n_xrows;
        const size_t lds = (size_t)xr * xs_bytes(K);
        if (lds <= 64 * 1024) {
            pl.lpr = lpr, pl.deep = deep, pl.lds = lds;
            return true;
        }
        if (lpr >= 64) return false;
    }
}

template <int QT, bool SW>
int launch_idv(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
               int n_pairs, int top_k, int n_xrows, float* Y, size_t ldy, int N, int K, const float* sc, int* err,
               int lpr, int wgs_per_cu, int deep, hipStream_t st) {
    if (lpr <= 0) lpr = pick_lpr_idv(K / 64, (long)n_pairs * N);
#define QMV_IDV_CASE(L)                                                                                          \
    if (lpr == L)                                                                                                \
        return launch_idv_t<QT, L, SW>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, n_xrows, Y, ldy, N, K, sc, err, \
                                       wgs_per_cu, deep, st);
    QMV_IDV_CASE(64) QMV_IDV_CASE(32) QMV_IDV_CASE(16) QMV_IDV_CASE(8) QMV_IDV_CASE(4)
#undef QMV_IDV_CASE
    return fail(QMV_EINVAL, "internal: no few-pairs id kernel for lpr=%d", lpr);
}

template <int QT, bool SW>
int launch_id(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
              int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err, int fast,
              hipStream_t st) {
    const int lpr = fast ? pick_lpr(K / 64) : 64;
#define QMV_ID_CASE(L) \
    if (lpr == L) return launch_id_t<QT, L, 1, SW>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, fast, st);
    QMV_ID_CASE(64) QMV_ID_CASE(32) QMV_ID_CASE(16) QMV_ID_CASE(8) QMV_ID_CASE(4)
#undef QMV_ID_CASE
    return fail(QMV_EINVAL, "internal: no id kernel for lpr=%d", lpr);
}

int launch_id_q6(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
                 int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err, int qtype,
                 hipStream_t st);

// Shared by qmv_id (SW = false: X rows hold K values) and qmv_id_swiglu
// (SW = true: X rows hold 2K values, gate then up). `fn` names the entry point
// in error messages.
template <bool SW>
int id_common(const char* fn, int qtype, const void* Wv, size_t expert_stride_bytes, size_t ldw_bytes, int n_experts,
              const float* X, size_t ldx, const uint32_t* ids, int n_tokens, int top_k, float* Y, size_t ldy, int N,
              int K, const float* expert_scale, int* err_flag, void* stream) {
    const bool q6 = qtype == QMV_Q6_K || qtype == QMV_Q5_K;  // super-block formats
    if (qtype != QMV_Q4_0 && qtype != QMV_Q8_0 && !(q6 && !SW))
        return fail(QMV_EUNSUPPORTED, "%s: qtype %d not supported", fn, qtype);
    const int bb = qtype == QMV_Q6_K ? Q6_SB_BYTES : qtype == QMV_Q5_K ? Q5_SB_BYTES : block_bytes(qtype);
    const int qk = q6 ? 256 : QK;
    if (n_experts <= 0) return fail(QMV_EINVAL, "%s: n_experts=%d must be > 0", fn, n_experts);
    if (top_k <= 0) return fail(QMV_EINVAL, "%s: top_k=%d must be > 0", fn, top_k);
    if (n_tokens < 0) return fail(QMV_EINVAL, "%s: n_tokens=%d < 0", fn, n_tokens);
    if (N < 0) return fail(QMV_EINVAL, "%s: N=%d < 0", fn, N);
    if (K < 0 || K % qk) return fail(QMV_EINVAL, "%s: K=%d is not a non-negative multiple of %d", fn, K, qk);
    if (q6 && K > KMAX_Q6) return fail(QMV_EUNSUPPORTED, "%s: K=%d exceeds %d for Q6_K and Q5_K", fn, K, KMAX_Q6);
    if (top_k > ID_MAX_LIST) return fail(QMV_EUNSUPPORTED, "%s: top_k=%d exceeds %d", fn, top_k, ID_MAX_LIST);
    if ((long)n_tokens * top_k > 0x7FFFFFFFL) return fail(QMV_EINVAL, "%s: n_tokens*top_k overflows", fn);
    if (n_tokens == 0 || N == 0) return QMV_OK;
    if (!Wv || !X || !ids || !Y) return fail(QMV_EINVAL, "%s: NULL W, X, ids or Y", fn);
    const size_t row = (size_t)(K / qk) * bb;
    if (ldw_bytes < row) return fail(QMV_EINVAL, "%s: ldw_bytes=%zu < K/%d*%d=%zu", fn, ldw_bytes, qk, bb, row);
    if ((size_t)N > SIZE_MAX / (ldw_bytes ? ldw_bytes : 1)) return fail(QMV_EINVAL, "%s: N*ldw overflows", fn);
    if (expert_stride_bytes < (size_t)N * ldw_bytes)
        return fail(QMV_EINVAL, "%s: expert_stride_bytes=%zu < N*ldw_bytes=%zu", fn, expert_stride_bytes,
                    (size_t)N * ldw_bytes);
    if (ldx < (size_t)(SW ? 2 : 1) * K)
        return fail(QMV_EINVAL, "%s: ldx=%zu < %s=%d", fn, ldx, SW ? "2K" : "K", (SW ? 2 : 1) * K);
    if (ldy < (size_t)N) return fail(QMV_EINVAL, "%s: ldy=%zu < N=%d", fn, ldy, N);
    if (((uintptr_t)Wv & 1) || (ldw_bytes & 1) || (expert_stride_bytes & 1))
        return fail(QMV_EALIGN, "%s: W, ldw_bytes and expert_stride_bytes must be 2-byte aligned", fn);
    if (((uintptr_t)X & 3) || ((uintptr_t)Y & 3) || ((uintptr_t)ids & 3) || ((uintptr_t)expert_scale & 3) ||
        ((uintptr_t)err_flag & 3))
        return fail(QMV_EALIGN, "%s: X, Y, ids, expert_scale and err_flag must be 4-byte aligned", fn);
    const int n_pairs = n_tokens * top_k;
    const size_t ybytes = ((size_t)(n_pairs - 1) * ldy + N) * 4;
    const size_t wbytes = (size_t)(n_experts - 1) * expert_stride_bytes + (size_t)(N - 1) * ldw_bytes + row;
    const size_t xbytes = ((size_t)(n_tokens - 1) * ldx + (size_t)(SW ? 2 : 1) * K) * 4;
    if (overlaps(Y, ybytes, Wv, K ? wbytes : 0) || overlaps(Y, ybytes, X, K ? xbytes : 0) ||
        overlaps(Y, ybytes, ids, (size_t)n_pairs * 4) ||
        overlaps(Y, ybytes, expert_scale, expert_scale ? (size_t)n_experts * 4 : 0) ||
        overlaps(Y, ybytes, err_flag, err_flag ? 4 : 0))
        return fail(QMV_EINVAL, "%s: Y overlaps another argument", fn);

    hipStream_t st = (hipStream_t)stream;
    const uint8_t* W = (const uint8_t*)Wv;
    if (q6 && K > 0)
        return launch_id_q6(W, expert_stride_bytes, ldw_bytes, n_experts, X, ldx, ids, n_tokens * top_k, top_k, Y,
                            ldy, N, K, expert_scale, err_flag, qtype, st);
    // (K = 0 of any type: the generic kernel reads no weights and writes zeros)
    const int fast = K > 0 && K % 64 == 0 && K <= KMAX_FAST_ID && ((uintptr_t)W & 3) == 0 && (ldw_bytes & 3) == 0 &&
                     ldw_bytes <= 0xFFFFFFFFu &&
                     (expert_stride_bytes & 3) == 0;
    // Up to 64 pairs (decode and short batches): stream all pairs' rows as
    // one matrix. Measured against the grouped kernel on the MoE calls
    // (128 experts, top-8): faster at T = 1, 2, 4 and 8 although experts
    // shared by several pairs are read once per pair.
    const int n_pairs_all = n_tokens * top_k;
    IdvPlan pl;
    if (fast && n_pairs_all <= IDV_MAX_PAIRS && (long)n_pairs_all * N < 0x7FFFFFFFL &&
        plan_idv(qtype, K, n_pairs_all, N, n_tokens, pl)) {
        return qtype == QMV_Q4_0
                   ? launch_idv<QMV_Q4_0, SW>(W, expert_stride_bytes, ldw_bytes, n_experts, X, ldx, ids, n_pairs_all,
                                              top_k, n_tokens, Y, ldy, N, K, expert_scale, err_flag, pl.lpr, 0,
                                              pl.deep, st)
                   : launch_idv<QMV_Q8_0, SW>(W, expert_stride_bytes, ldw_bytes, n_experts, X, ldx, ids, n_pairs_all,
                                              top_k, n_tokens, Y, ldy, N, K, expert_scale, err_flag, pl.lpr, 0,
                                              pl.deep, st);
    }
    // A launch groups at most ID_MAX_LIST pairs (the grouped kernel's lists,
    // the generic kernel's leader), so a call is split into launches over
    // whole tokens holding at most that many pairs each.
    static_assert(IDP_MAX_PAIRS == ID_MAX_LIST, "one pair limit per launch");
    const int tok_per_launch = ID_MAX_LIST / top_k;
    for (int t0 = 0; t0 < n_tokens; t0 += tok_per_launch) {
        const int nt = n_tokens - t0 < tok_per_launch ? n_tokens - t0 : tok_per_launch;
        const size_t p0 = (size_t)t0 * top_k;
        const float* Xs = X + (size_t)t0 * ldx;
        const uint32_t* is = ids + p0;
        float* Ys = Y + p0 * ldy;
        const bool grouped = fast && n_experts <= IDP_MAX_EXPERTS;
        // Grouped on the matrix cores when experts serve several pairs each
        // (at least 4 per expert on average): a 16-row MFMA block then holds
        // enough pairs to beat one FMA per weight and pair. Measured on the
        // MoE calls (128 experts, top-8): 1.6x faster than the vector kernel
        // at 128 and 256 tokens, slower at 32 (2 pairs per expert).
        const bool mfma = grouped && !SW && K >= 256 && (long)nt * top_k >= 4L * n_experts &&
                          ((uintptr_t)Xs & 15) == 0 && (ldx & 3) == 0 &&
                          ((size_t)(nt - 1) * ldx + (size_t)K) * 4 < 0x80000000u;  // X by 32-bit offsets
        int rc;
        if (mfma)
            rc = launch_idq(qtype, W, expert_stride_bytes, ldw_bytes, n_experts, Xs, ldx, is, nt * top_k, top_k, Ys, ldy,
                            N, K, expert_scale, err_flag, st);
        else if (grouped)
            rc = qtype == QMV_Q4_0
                     ? launch_idp<QMV_Q4_0, SW>(W, expert_stride_bytes, ldw_bytes, n_experts, Xs, ldx, is, nt * top_k,
                                                top_k, Ys, ldy, N, K, expert_scale, err_flag, st)
                     : launch_idp<QMV_Q8_0, SW>(W, expert_stride_bytes, ldw_bytes, n_experts, Xs, ldx, is, nt * top_k,
                                                top_k, Ys, ldy, N, K, expert_scale, err_flag, st);
        else
            rc = qtype == QMV_Q4_0
                     ? launch_id<QMV_Q4_0, SW>(W, expert_stride_bytes, ldw_bytes, n_experts, Xs, ldx, is, nt * top_k,
                                               top_k, Ys, ldy, N, K, expert_scale, err_flag, fast, st)
                     : launch_id<QMV_Q8_0, SW>(W, expert_stride_bytes, ldw_bytes, n_experts, Xs, ldx, is, nt * top_k,
                                               top_k, Ys, ldy, N, K, expert_scale, err_flag, fast, st);
        if (rc) return rc;
    }
    return QMV_OK;
}


template <int QT, int LPR, int WAVES>
int launch_moe_down_t(const uint8_t* W, size_t es, size_t ldw, int E, const float* G, size_t ldg, const uint32_t* ids,
                      const float* wts, int n_tokens, int top_k, float* out, size_t ldo, int N, int K,
                      const float* sc, int* err, hipStream_t st) {
    constexpr int R = 64 / LPR;
    const long tiles = ((long)N + R - 1) / R;
    if (tiles > 0x7FFFFFFF) return fail(QMV_EINVAL, "qmv_moe_down: N too large");
    const size_t lds = (size_t)top_k * xs_bytes(K);
    // grid.y is limited to 65535: launch over slices of the tokens.
    for (int t0 = 0; t0 < n_tokens; t0 += 65535) {
        const int nt = n_tokens - t0 < 65535 ? n_tokens - t0 : 65535;
        hipLaunchKernelGGL((k_moe_down<QT, LPR, WAVES>), dim3((unsigned)tiles, (unsigned)nt), dim3(WAVES * 64), lds, st,
                           W, es, ldw, E, G + (size_t)t0 * top_k * ldg, ldg, ids + (size_t)t0 * top_k,
                           wts + (size_t)t0 * top_k, top_k, out + (size_t)t0 * ldo, ldo, N, K, sc, err);
        const int rc = check_launch("qmv_moe_down kernel");
        if (rc) return rc;
    }
    return QMV_OK;
}

template <int QT, int WAVES>
int launch_moe_down_w(const uint8_t* W, size_t es, size_t ldw, int E, const float* G, size_t ldg, const uint32_t* ids,
                      const float* wts, int n_tokens, int top_k, float* out, size_t ldo, int N, int K,
                      const float* sc, int* err, hipStream_t st) {
    const int lpr = pick_lpr(K / 64);
#define QMV_MD_CASE(L)                                                                                            \
    if (lpr == L)                                                                                                 \
        return launch_moe_down_t<QT, L, WAVES>(W, es, ldw, E, G, ldg, ids, wts, n_tokens, top_k, out, ldo, N, K, sc, \
                                               err, st);
    QMV_MD_CASE(64) QMV_MD_CASE(32) QMV_MD_CASE(16) QMV_MD_CASE(8) QMV_MD_CASE(4)
#undef QMV_MD_CASE
    return fail(QMV_EINVAL, "internal: no moe_down kernel for lpr=%d", lpr);
}

// Waves per workgroup: one per slot up to 8.
template <int QT>
int launch_moe_down(const uint8_t* W, size_t es, size_t ldw, int E, const float* G, size_t ldg, const uint32_t* ids,
                    const float* wts, int n_tokens, int top_k, float* out, size_t ldo, int N, int K, const float* sc,
                    int* err, hipStream_t st) {
    if (top_k <= 2)
        return launch_moe_down_w<QT, 2>(W, es, ldw, E, G, ldg, ids, wts, n_tokens, top_k, out, ldo, N, K, sc, err, st);
    if (top_k <= 4)
        return launch_moe_down_w<QT, 4>(W, es, ldw, E, G, ldg, ids, wts, n_tokens, top_k, out, ldo, N, K, sc, err, st);
    return launch_moe_down_w<QT, 8>(W, es, ldw, E, G, ldg, ids, wts, n_tokens, top_k, out, ldo, N, K, sc, err, st);
}

constexpr size_t MD_LDS_MAX = 64 * 1024;  // staged SwiGLU rows of one token

// Separate per-group scales and biases of the affine format (unused by the
// super-block formats): row n's at S + n * lds, expert e's block s_estride
// elements after expert e - 1's.
struct AuxArgs {
    const uint16_t* S = nullptr;
    const uint16_t* B = nullptr;
    size_t lds = 0, s_estride = 0;
};

template <class F, int LPR, int WAVES, int MX>
int launch_q6k_t(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int nx, int N, int K,
                 int wgs_per_cu, hipStream_t st, const AuxArgs& ax) {
    constexpr int ROWS = (64 / LPR) * WAVES;
    const long tiles = ((long)N + ROWS - 1) / ROWS;
    long nwg = (long)num_cus() * (wgs_per_cu > 0 ? wgs_per_cu : 2);
    nwg = nwg < tiles ? nwg : tiles;
    const size_t lds = (size_t)nx * q6_xs_bytes(K);
    hipLaunchKernelGGL((k_q6k<F, LPR, WAVES, MX>), dim3((unsigned)nwg), dim3(WAVES * 64), lds, st, W, ldw, X, ldx, Y,
                       ldy, nx, N, K, ax.S, ax.B, ax.lds);
    return check_launch("super-block kernel");
}

template <class F, int LPR>
int launch_id_q6_t(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
                   int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err,
                   hipStream_t st, const AuxArgs& ax) {
    constexpr int WAVES = 4;
    constexpr int ROWS = (64 / LPR) * WAVES;
    const long tiles = ((long)N + ROWS - 1) / ROWS;
    if (tiles > 0x7FFFFFFF) return fail(QMV_EINVAL, "qmv_id: N too large");
    // grid.y holds at most 65535 pairs: launches over whole tokens
    const int per = (65535 / top_k) * top_k;
    for (int p0 = 0; p0 < n_pairs; p0 += per) {
        const int np = n_pairs - p0 < per ? n_pairs - p0 : per;
        hipLaunchKernelGGL((k_id_q6<F, LPR, WAVES>), dim3((unsigned)tiles, (unsigned)np), dim3(WAVES * 64),
                           q6_xs_bytes(K), st, W, es, ldw, E, X + (size_t)(p0 / top_k) * ldx, ldx, ids + p0, top_k,
                           Y + (size_t)p0 * ldy, ldy, N, K, sc, err, ax.S, ax.B, ax.s_estride, ax.lds);
        const int rc = check_launch("qmv_id super-block kernel");
        if (rc) return rc;
    }
    return QMV_OK;
}

template <class F>
int launch_id_kq(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
                 int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err,
                 hipStream_t st, const AuxArgs& ax = AuxArgs{}) {
    const int lpr = pick_lpr_q6(F::units(K));
#define QMV_IDQ6_CASE(L)                                                                                            \
    if (lpr == L)                                                                                                   \
        return launch_id_q6_t<F, L>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, st, ax);
    QMV_IDQ6_CASE(64) QMV_IDQ6_CASE(32) QMV_IDQ6_CASE(16) QMV_IDQ6_CASE(8) QMV_IDQ6_CASE(4)
#undef QMV_IDQ6_CASE
    return fail(QMV_EINVAL, "internal: no super-block id kernel for lpr=%d", lpr);
}

int launch_id_q6(const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx, const uint32_t* ids,
                 int n_pairs, int top_k, float* Y, size_t ldy, int N, int K, const float* sc, int* err, int qtype,
                 hipStream_t st) {
    return qtype == QMV_Q5_K ? launch_id_kq<FmtQ5K>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, st)
                             : launch_id_kq<FmtQ6K>(W, es, ldw, E, X, ldx, ids, n_pairs, top_k, Y, ldy, N, K, sc, err, st);
}

// Batched M = 1 super-block products sharing x and K (k_q6kc): lane groups
// widened until there are two tiles per compute unit (the B9 group, 11648
// rows of K = 2816 in Q5_K: 32 lanes per row 11.4 us; 16 lanes, one tile per
// unit, 13.4 us; 64 lanes 17.0 us).
template <class F, int LPR, int MAXP>
int launch_q6kc_t(const M1Prob* probs, int n, hipStream_t st) {
    constexpr int WAVES = 8, ROWS = (64 / LPR) * WAVES;
    Q6Cat<MAXP> C{};
    long t = 0;
    for (int i = 0; i < n; ++i) {
        C.W[i] = probs[i].W;
        C.ldw[i] = probs[i].ldw;
        C.y[i] = probs[i].y;
        C.N[i] = probs[i].N;
        C.t0[i] = t;
        t += ((long)probs[i].N + ROWS - 1) / ROWS;
    }
    C.t0[n] = t;
    C.x = probs[0].x;
    C.K = probs[0].K;
    C.n = n;
    if (t > 0x7FFFFFFF) return fail(QMV_EINVAL, "qmv_batch: N too large");  // tile indices are 32-bit
    long nwg = (long)num_cus() * 2;
    nwg = nwg < t ? nwg : t;
    hipLaunchKernelGGL((k_q6kc<F, LPR, WAVES, MAXP>), dim3((unsigned)nwg), dim3(WAVES * 64), q6_xs_bytes(C.K), st, C);
    return check_launch("batched super-block kernel");
}

template <class F, int MAXP>
int launch_q6kc_n(const M1Prob* probs, int n, hipStream_t st) {
    long rows = 0;
    for (int i = 0; i < n; ++i) rows += probs[i].N;
    int lpr = pick_lpr_q6(F::units(probs[0].K));
    while (lpr < 64 && (rows + (64 / lpr) * 8 - 1) / ((64 / lpr) * 8) < 2 * num_cus()) lpr *= 2;
    switch (lpr) {
        case 64: return launch_q6kc_t<F, 64, MAXP>(probs, n, st);
        case 32: return launch_q6kc_t<F, 32, MAXP>(probs, n, st);
        case 16: return launch_q6kc_t<F, 16, MAXP>(probs, n, st);
        case 8: return launch_q6kc_t<F, 8, MAXP>(probs, n, st);
        default: return launch_q6kc_t<F, 4, MAXP>(probs, n, st);
    }
}

template <class F>
int launch_q6kc(const M1Prob* probs, int n, hipStream_t st) {
    return n <= 4 ? launch_q6kc_n<F, 4>(probs, n, st) : launch_q6kc_n<F, QMV_MAX_BATCH>(probs, n, st);
}

// Rows of X in launches of up to 4 (one launch when M = 1).
template <class F>
int launch_q6k(const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
               int lpr, int wgs_per_cu, hipStream_t st, const AuxArgs& ax = AuxArgs{}) {
    if (lpr <= 0) {
        // widen the lane groups of short calls until every compute unit has
        // a tile (5760 rows at 8 lanes per row are 90 tiles of 64 rows)
        lpr = pick_lpr_q6(F::units(K));
        while (lpr < 64 && ((long)N + (64 / lpr) * 8 - 1) / ((64 / lpr) * 8) < num_cus()) lpr *= 2;
    }
    for (int m0 = 0; m0 < M; m0 += 4) {
        const int nx = M - m0 < 4 ? M - m0 : 4;
        const float* Xm = X + (size_t)m0 * ldx;
        float* Ym = Y + (size_t)m0 * ldy;
        int rc = QMV_EINVAL;
#define QMV_Q6_CASE(L)                                                                                   \
    if (lpr == L)                                                                                        \
        rc = nx == 1 ? launch_q6k_t<F, L, 8, 1>(W, ldw, Xm, ldx, Ym, ldy, 1, N, K, wgs_per_cu, st, ax)   \
                     : launch_q6k_t<F, L, 8, 4>(W, ldw, Xm, ldx, Ym, ldy, nx, N, K, wgs_per_cu, st, ax);
        QMV_Q6_CASE(64) QMV_Q6_CASE(32) QMV_Q6_CASE(16) QMV_Q6_CASE(8) QMV_Q6_CASE(4)
#undef QMV_Q6_CASE
        if (rc) return rc == QMV_EINVAL ? fail(QMV_EINVAL, "internal: no super-block kernel for lpr=%d", lpr) : rc;
    }
    return QMV_OK;
}
// Dense call of a super-block format (shared by qmv_q5_k and qmv_q6_k).
template <class F>
int kq_dense(const char* name, const void* Wv, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M,
             int N, int K, void* stream) {
    if (M < 0 || M > QMV_MAX_M) return fail(QMV_EUNSUPPORTED, "%s: M=%d outside 0..%d", name, M, QMV_MAX_M);
    if (N < 0) return fail(QMV_EINVAL, "%s: N=%d < 0", name, N);
    if (K < 0 || K % 256) return fail(QMV_EINVAL, "%s: K=%d is not a non-negative multiple of 256", name, K);
    if (M == 0 || N == 0) return QMV_OK;
    if (!Wv && K > 0) return fail(QMV_EINVAL, "%s: W is NULL", name);
    if (!X && K > 0) return fail(QMV_EINVAL, "%s: X is NULL", name);
    if (!Y) return fail(QMV_EINVAL, "%s: Y is NULL", name);
    if (K > KMAX_Q6) return fail(QMV_EUNSUPPORTED, "%s: K=%d exceeds %d", name, K, KMAX_Q6);
    const size_t row = (size_t)(K / 256) * F::SB;
    if (ldw < row) return fail(QMV_EINVAL, "%s: ldw_bytes=%zu < K/256*%d=%zu", name, ldw, F::SB, row);
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
    if (K == 0)  // empty sums: the generic kernel reads no weights and writes zeros
        return launch_generic<QMV_Q4_0>((const uint8_t*)Wv, ldw, X, ldx, Y, ldy, M, N, 0, st);
    return launch_q6k<F>((const uint8_t*)Wv, ldw, X, ldx, Y, ldy, M, N, K, 0, 0, st);
}

// ---------------------------------------------------------------------------
// Streaming-read reference for measurements: every 16-byte chunk of a buffer
// read once with non-temporal loads (the pattern closest to HBM peak here),
// eight per thread in flight, XOR-folded. A word is written to sink only if
// a workgroup's fold equals a constant that the data never produces in
// practice, so that the loads cannot be dropped; the write does not matter.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ src, size_t n16, uint32_t* sink) {
    constexpr int U = 8;
    const size_t chunk = (size_t)256 * U;
    const size_t nch = n16 / chunk;
    uint32_t acc = 0;
    for (size_t c = blockIdx.x; c < nch; c += gridDim.x) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + c * chunk + u * 256 + threadIdx.x);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // the tail (fewer than 256 * U chunks of 16 bytes) by workgroup 0
    if (blockIdx.x == 0)
        for (size_t i = nch * chunk + threadIdx.x; i < n16; i += 256) {
            const u32x4 t = src[i];
            acc ^= t.x ^ t.y ^ t.z ^ t.w;
        }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch for qmv_ws_static: the K-segment partial sums of qmv_ws kept
// in the library's own device memory (one copy per GPU, held until the
// process ends), for callers that cannot allocate. Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current);
// host code passes that address to the kernels, never the symbol itself.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[QMV_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch_ptr[MAX_DEVICES];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (nullptr and the error message
// set if it cannot be had).
void* static_scratch(const char* name) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        (void)hipGetLastError();
        fail(QMV_EHIP, "%s: no current device (or device id >= %d)", name, MAX_DEVICES);
        return nullptr;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            fail(QMV_EHIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", name, dev,
                 hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
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

size_t qmv_ws_bytes(int qtype, int M, int N, int K) {
    if ((qtype != QMV_Q4_0 && qtype != QMV_Q8_0) || M < 2 || M > QMV_MAX_M || N <= 0 || K <= 0 || K % 64) return 0;
    return mq_ws_bytes(M, N, K);
}

int qmv_ws(int qtype, const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N,
           int K, void* workspace, size_t workspace_bytes, void* stream) {
    if (qtype != QMV_Q4_0 && qtype != QMV_Q8_0) return fail(QMV_EUNSUPPORTED, "qmv_ws: qtype %d not supported", qtype);
    const size_t need = qmv_ws_bytes(qtype, M, N, K);
    if (workspace && workspace_bytes < need)
        return fail(QMV_EINVAL, "qmv_ws: workspace_bytes=%zu < %zu needed for M=%d N=%d K=%d", workspace_bytes, need, M,
                    N, K);
    return dense(qtype, W, ldw_bytes, X, ldx, Y, ldy, M, N, K, stream, workspace, workspace ? workspace_bytes : 0,
                 "qmv_ws");
}

int qmv_ws_static(int qtype, const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy, int M,
                  int N, int K, void* stream) {
    if (qtype != QMV_Q4_0 && qtype != QMV_Q8_0)
        return fail(QMV_EUNSUPPORTED, "qmv_ws_static: qtype %d not supported", qtype);
    const size_t need = qmv_ws_bytes(qtype, M, N, K);
    if (need > (size_t)QMV_STATIC_SCRATCH_BYTES)
        return fail(QMV_EINVAL,
                    "qmv_ws_static: M=%d N=%d K=%d needs %zu bytes of scratch, more than the static %d; use qmv_ws "
                    "with a workspace",
                    M, N, K, need, QMV_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0 && !(ws = static_scratch("qmv_ws_static"))) return QMV_EHIP;
    return dense(qtype, W, ldw_bytes, X, ldx, Y, ldy, M, N, K, stream, ws, ws ? (size_t)QMV_STATIC_SCRATCH_BYTES : 0,
                 "qmv_ws_static");
}

int qmv_id(int qtype, const void* Wv, size_t expert_stride_bytes, size_t ldw_bytes, int n_experts, const float* X,
           size_t ldx, const uint32_t* ids, int n_tokens, int top_k, float* Y, size_t ldy, int N, int K,
           const float* expert_scale, int* err_flag, void* stream) {
    return id_common<false>("qmv_id", qtype, Wv, expert_stride_bytes, ldw_bytes, n_experts, X, ldx, ids, n_tokens,
                            top_k, Y, ldy, N, K, expert_scale, err_flag, stream);
}

int qmv_id_swiglu(int qtype, const void* Wv, size_t expert_stride_bytes, size_t ldw_bytes, int n_experts,
                  const float* G, size_t ldg, const uint32_t* ids, int n_tokens, int top_k, float* Y, size_t ldy,
                  int N, int K, const float* expert_scale, int* err_flag, void* stream) {
    return id_common<true>("qmv_id_swiglu", qtype, Wv, expert_stride_bytes, ldw_bytes, n_experts, G, ldg, ids,
                           n_tokens, top_k, Y, ldy, N, K, expert_scale, err_flag, stream);
}

int qmv_q5_k(const void* Wv, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
             void* stream) {
    return kq_dense<FmtQ5K>("qmv_q5_k", Wv, ldw, X, ldx, Y, ldy, M, N, K, stream);
}

int qmv_q6_k(const void* Wv, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K,
             void* stream) {
    return kq_dense<FmtQ6K>("qmv_q6_k", Wv, ldw, X, ldx, Y, ldy, M, N, K, stream);
}

// Activation rows from which qmv_gemm takes the tiled kernel (its tiles are
// 128 rows; below this the 16-row blocks of k_mq waste less).
constexpr int GEMM_MIN_M = 64;

int qmv_gemm(int qtype, const void* Wv, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy, int M, int N,
             int K, void* stream) {
    const char* name = "qmv_gemm";
    const bool kq = qtype == QMV_Q6_K || qtype == QMV_Q5_K;
    if (qtype != QMV_Q4_0 && qtype != QMV_Q8_0 && !kq)
        return fail(QMV_EUNSUPPORTED, "%s: qtype %d not supported", name, qtype);
    const int qk = kq ? 256 : QK;
    const int bb = qtype == QMV_Q6_K ? Q6_SB_BYTES : qtype == QMV_Q5_K ? Q5_SB_BYTES : block_bytes(qtype);
    if (M < 0) return fail(QMV_EINVAL, "%s: M=%d < 0", name, M);
    if (N < 0) return fail(QMV_EINVAL, "%s: N=%d < 0", name, N);
    if (K < 0 || K % qk) return fail(QMV_EINVAL, "%s: K=%d is not a non-negative multiple of %d", name, K, qk);
    if (M == 0 || N == 0) return QMV_OK;
    if ((!Wv || !X) && K > 0) return fail(QMV_EINVAL, "%s: W or X is NULL", name);
    if (!Y) return fail(QMV_EINVAL, "%s: Y is NULL", name);
    const size_t row = (size_t)(K / qk) * bb;
    if (ldw < row) return fail(QMV_EINVAL, "%s: ldw_bytes=%zu < K/%d*%d=%zu", name, ldw, qk, bb, row);
    if (M > 1 && ldx < (size_t)K) return fail(QMV_EINVAL, "%s: ldx=%zu < K=%d", name, ldx, K);
    if (M > 1 && ldy < (size_t)N) return fail(QMV_EINVAL, "%s: ldy=%zu < N=%d", name, ldy, N);
    if (((uintptr_t)Wv & 1) || (ldw & 1)) return fail(QMV_EALIGN, "%s: W and ldw_bytes must be 2-byte aligned", name);
    if (((uintptr_t)X & 3) || ((uintptr_t)Y & 3)) return fail(QMV_EALIGN, "%s: X and Y must be 4-byte aligned", name);
    if (M == 1) ldx = (size_t)K, ldy = (size_t)N;
    if ((size_t)N > (SIZE_MAX - row) / (ldw ? ldw : 1)) return fail(QMV_EINVAL, "%s: N*ldw overflows", name);
    if ((size_t)M > (SIZE_MAX / 4 - (size_t)N) / (ldy ? ldy : 1)) return fail(QMV_EINVAL, "%s: M*ldy overflows", name);
    const size_t wbytes = K ? (size_t)(N - 1) * ldw + row : 0;
    const size_t xbytes = K ? ((size_t)(M - 1) * ldx + K) * 4 : 0;
    const size_t ybytes = ((size_t)(M - 1) * ldy + N) * 4;
    if (overlaps(Y, ybytes, Wv, wbytes) || overlaps(Y, ybytes, X, xbytes))
        return fail(QMV_EINVAL, "%s: Y overlaps W or X", name);
    // Q4_0 and Q8_0 with at least GEMM_MIN_M rows and 16-byte aligned rows of
    // X: tiles of 64 x 256 outputs, each weight decoded once per 64 rows.
    // Otherwise every block of 16 rows in one matrix-core launch (blocks that
    // read the same weights run side by side and share them through L2).
    const bool q = (qtype == QMV_Q4_0 || qtype == QMV_Q8_0) && K > 0 && K % 64 == 0 && ((uintptr_t)Wv & 3) == 0 &&
                   (ldw & 3) == 0;
    if (q && M >= GEMM_MIN_M && ldw <= 0xFFFFFFFFu && ((uintptr_t)X & 15) == 0 && (ldx & 3) == 0)
        return launch_gemm(qtype, (const uint8_t*)Wv, ldw, X, ldx, Y, ldy, M, N, K, (hipStream_t)stream);
    if (q && M > QMV_MAX_M)
        return launch_mq(qtype, (const uint8_t*)Wv, ldw, X, ldx, Y, ldy, M, N, K, nullptr, 0, (hipStream_t)stream);
    // Blocks of up to 16 activation rows, each through the dense call of its
    // type (matrix cores for Q4_0); every block reads the weights once.
    for (int m0 = 0; m0 < M; m0 += QMV_MAX_M) {
        const int mb = M - m0 < QMV_MAX_M ? M - m0 : QMV_MAX_M;
        const float* Xm = X + (size_t)m0 * ldx;
        float* Ym = Y + (size_t)m0 * ldy;
        int rc;
        if (qtype == QMV_Q6_K)
            rc = kq_dense<FmtQ6K>(name, Wv, ldw, Xm, ldx, Ym, ldy, mb, N, K, stream);
        else if (qtype == QMV_Q5_K)
            rc = kq_dense<FmtQ5K>(name, Wv, ldw, Xm, ldx, Ym, ldy, mb, N, K, stream);
        else
            rc = dense(qtype, Wv, ldw, Xm, ldx, Ym, ldy, mb, N, K, stream);
        if (rc) return rc;
    }
    return QMV_OK;
}

int qmv_affine4(const uint32_t* Wq, size_t ldw, const uint16_t* scales, const uint16_t* biases, size_t lds,
                const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K, void* stream) {
    const char* name = "qmv_affine4";
    if (M < 0 || M > QMV_MAX_M) return fail(QMV_EUNSUPPORTED, "%s: M=%d outside 0..%d", name, M, QMV_MAX_M);
    if (N < 0) return fail(QMV_EINVAL, "%s: N=%d < 0", name, N);
    if (K < 0 || K % 32) return fail(QMV_EINVAL, "%s: K=%d is not a non-negative multiple of 32", name, K);
    if (M == 0 || N == 0) return QMV_OK;
    if (K == 0) return fail(QMV_EUNSUPPORTED, "%s: K=0", name);
    if (K > KMAX_Q6) return fail(QMV_EUNSUPPORTED, "%s: K=%d exceeds %d", name, K, KMAX_Q6);
    if (!Wq || !scales || !biases || !X || !Y) return fail(QMV_EINVAL, "%s: NULL argument", name);
    if (ldw < (size_t)K / 8) return fail(QMV_EINVAL, "%s: ldw=%zu words < K/8=%d", name, ldw, K / 8);
    if (lds < (size_t)K / 32) return fail(QMV_EINVAL, "%s: lds=%zu < K/32=%d", name, lds, K / 32);
    if (M > 1 && ldx < (size_t)K) return fail(QMV_EINVAL, "%s: ldx=%zu < K=%d", name, ldx, K);
    if (M > 1 && ldy < (size_t)N) return fail(QMV_EINVAL, "%s: ldy=%zu < N=%d", name, ldy, N);
    if (((uintptr_t)Wq & 3) || ((uintptr_t)X & 3) || ((uintptr_t)Y & 3) || ((uintptr_t)scales & 1) ||
        ((uintptr_t)biases & 1))
        return fail(QMV_EALIGN, "%s: Wq, X and Y must be 4-byte aligned, scales and biases 2-byte", name);
    if (M == 1) ldx = (size_t)K, ldy = (size_t)N;
    if ((size_t)N > SIZE_MAX / 4 / (ldw > lds ? ldw : lds)) return fail(QMV_EINVAL, "%s: N*ldw overflows", name);
    const size_t ybytes = ((size_t)(M - 1) * ldy + N) * 4;
    const size_t sbytes = ((size_t)(N - 1) * lds + K / 32) * 2;
    if (overlaps(Y, ybytes, Wq, ((size_t)(N - 1) * ldw + K / 8) * 4) || overlaps(Y, ybytes, X, ((size_t)(M - 1) * ldx + K) * 4) ||
        overlaps(Y, ybytes, scales, sbytes) || overlaps(Y, ybytes, biases, sbytes))
        return fail(QMV_EINVAL, "%s: Y overlaps an input", name);
    AuxArgs ax;
    ax.S = scales, ax.B = biases, ax.lds = lds;
    return launch_q6k<FmtA4>((const uint8_t*)Wq, ldw * 4, X, ldx, Y, ldy, M, N, K, 0, 0, (hipStream_t)stream, ax);
}

int qmv_affine4_id(const uint32_t* Wq, size_t expert_stride_words, size_t ldw, const uint16_t* scales,
                   const uint16_t* biases, size_t expert_stride_groups, size_t lds, int n_experts, const float* X,
                   size_t ldx, const uint32_t* ids, int n_tokens, int top_k, float* Y, size_t ldy, int N, int K,
                   const float* expert_scale, int* err_flag, void* stream) {
    const char* name = "qmv_affine4_id";
    if (n_experts <= 0) return fail(QMV_EINVAL, "%s: n_experts=%d must be > 0", name, n_experts);
    if (top_k <= 0) return fail(QMV_EINVAL, "%s: top_k=%d must be > 0", name, top_k);
    if (n_tokens < 0) return fail(QMV_EINVAL, "%s: n_tokens=%d < 0", name, n_tokens);
    if (N < 0) return fail(QMV_EINVAL, "%s: N=%d < 0", name, N);
    if (K < 0 || K % 32) return fail(QMV_EINVAL, "%s: K=%d is not a non-negative multiple of 32", name, K);
    if ((long)n_tokens * top_k > 0x7FFFFFFFL) return fail(QMV_EINVAL, "%s: n_tokens*top_k overflows", name);
    if (n_tokens == 0 || N == 0) return QMV_OK;
    if (K == 0) return fail(QMV_EUNSUPPORTED, "%s: K=0", name);
    if (K > KMAX_Q6) return fail(QMV_EUNSUPPORTED, "%s: K=%d exceeds %d", name, K, KMAX_Q6);
    if (!Wq || !scales || !biases || !X || !ids || !Y) return fail(QMV_EINVAL, "%s: NULL argument", name);
    if (ldw < (size_t)K / 8) return fail(QMV_EINVAL, "%s: ldw=%zu words < K/8=%d", name, ldw, K / 8);
    if (lds < (size_t)K / 32) return fail(QMV_EINVAL, "%s: lds=%zu < K/32=%d", name, lds, K / 32);
    if ((size_t)N > SIZE_MAX / 4 / (ldw > lds ? ldw : lds)) return fail(QMV_EINVAL, "%s: N*ldw overflows", name);
    if (expert_stride_words < (size_t)N * ldw)
        return fail(QMV_EINVAL, "%s: expert_stride_words=%zu < N*ldw", name, expert_stride_words);
    if (expert_stride_groups < (size_t)N * lds)
        return fail(QMV_EINVAL, "%s: expert_stride_groups=%zu < N*lds", name, expert_stride_groups);
    if (ldx < (size_t)K) return fail(QMV_EINVAL, "%s: ldx=%zu < K=%d", name, ldx, K);
    if (ldy < (size_t)N) return fail(QMV_EINVAL, "%s: ldy=%zu < N=%d", name, ldy, N);
    if (((uintptr_t)Wq & 3) || ((uintptr_t)X & 3) || ((uintptr_t)Y & 3) || ((uintptr_t)ids & 3) ||
        ((uintptr_t)expert_scale & 3) || ((uintptr_t)err_flag & 3) || ((uintptr_t)scales & 1) ||
        ((uintptr_t)biases & 1))
        return fail(QMV_EALIGN, "%s: Wq, X, Y, ids, expert_scale, err_flag 4-byte, scales and biases 2-byte", name);
    const int n_pairs = n_tokens * top_k;
    const size_t ybytes = ((size_t)(n_pairs - 1) * ldy + N) * 4;
    const size_t wbytes = ((size_t)(n_experts - 1) * expert_stride_words + (size_t)(N - 1) * ldw + K / 8) * 4;
    const size_t sbytes = ((size_t)(n_experts - 1) * expert_stride_groups + (size_t)(N - 1) * lds + K / 32) * 2;
    if (overlaps(Y, ybytes, Wq, wbytes) || overlaps(Y, ybytes, X, ((size_t)(n_tokens - 1) * ldx + K) * 4) ||
        overlaps(Y, ybytes, scales, sbytes) || overlaps(Y, ybytes, biases, sbytes) ||
        overlaps(Y, ybytes, ids, (size_t)n_pairs * 4) ||
        overlaps(Y, ybytes, expert_scale, expert_scale ? (size_t)n_experts * 4 : 0) ||
        overlaps(Y, ybytes, err_flag, err_flag ? 4 : 0))
        return fail(QMV_EINVAL, "%s: Y overlaps another argument", name);
    AuxArgs ax;
    ax.S = scales, ax.B = biases, ax.lds = lds, ax.s_estride = expert_stride_groups;
    return launch_id_kq<FmtA4>((const uint8_t*)Wq, expert_stride_words * 4, ldw * 4, n_experts, X, ldx, ids, n_pairs,
                               top_k, Y, ldy, N, K, expert_scale, err_flag, (hipStream_t)stream, ax);
}

int qmv_moe_wsum(const float* Y, size_t ldy, const float* weights, int n_tokens, int top_k, int N, float* out,
                 size_t ldo, void* stream) {
    if (n_tokens < 0) return fail(QMV_EINVAL, "qmv_moe_wsum: n_tokens=%d < 0", n_tokens);
    if (top_k <= 0) return fail(QMV_EINVAL, "qmv_moe_wsum: top_k=%d must be > 0", top_k);
    if (N < 0) return fail(QMV_EINVAL, "qmv_moe_wsum: N=%d < 0", N);
    if ((long)n_tokens * top_k > 0x7FFFFFFFL) return fail(QMV_EINVAL, "qmv_moe_wsum: n_tokens*top_k overflows");
    if (n_tokens == 0 || N == 0) return QMV_OK;
    if (!Y || !weights || !out) return fail(QMV_EINVAL, "qmv_moe_wsum: NULL Y, weights or out");
    if (ldy < (size_t)N) return fail(QMV_EINVAL, "qmv_moe_wsum: ldy=%zu < N=%d", ldy, N);
    if (ldo < (size_t)N) return fail(QMV_EINVAL, "qmv_moe_wsum: ldo=%zu < N=%d", ldo, N);
    if (((uintptr_t)Y & 3) || ((uintptr_t)weights & 3) || ((uintptr_t)out & 3))
        return fail(QMV_EALIGN, "qmv_moe_wsum: Y, weights and out must be 4-byte aligned");
    const size_t P = (size_t)n_tokens * top_k;
    const size_t obytes = ((size_t)(n_tokens - 1) * ldo + N) * 4;
    if (overlaps(out, obytes, Y, ((P - 1) * ldy + N) * 4) || overlaps(out, obytes, weights, P * 4))
        return fail(QMV_EINVAL, "qmv_moe_wsum: out overlaps another argument");
    const long col_tiles = ((long)N + 255) / 256;
    if ((long)n_tokens * col_tiles > 0x7FFFFFFFL) return fail(QMV_EINVAL, "qmv_moe_wsum: too many tokens x columns");
    hipLaunchKernelGGL(k_wsum, dim3((unsigned)(n_tokens * col_tiles)), dim3(256), 0, (hipStream_t)stream, Y, ldy,
                       weights, top_k, N, col_tiles, out, ldo);
    return check_launch("qmv_moe_wsum kernel");
}

int qmv_moe_down(int qtype, const void* Wv, size_t expert_stride_bytes, size_t ldw_bytes, int n_experts,
                 const float* G, size_t ldg, const uint32_t* ids, const float* weights, int n_tokens, int top_k,
                 float* out, size_t ldo, int N, int K, const float* expert_scale, int* err_flag, void* stream) {
    if (qtype != QMV_Q4_0 && qtype != QMV_Q8_0)
        return fail(QMV_EUNSUPPORTED, "qmv_moe_down: qtype %d not supported", qtype);
    const int bb = block_bytes(qtype);
    if (n_experts <= 0) return fail(QMV_EINVAL, "qmv_moe_down: n_experts=%d must be > 0", n_experts);
    if (top_k <= 0) return fail(QMV_EINVAL, "qmv_moe_down: top_k=%d must be > 0", top_k);
    if (n_tokens < 0) return fail(QMV_EINVAL, "qmv_moe_down: n_tokens=%d < 0", n_tokens);
    if (N < 0) return fail(QMV_EINVAL, "qmv_moe_down: N=%d < 0", N);
    if (K < 0 || K % QK) return fail(QMV_EINVAL, "qmv_moe_down: K=%d is not a non-negative multiple of 32", K);
    if ((long)n_tokens * top_k > 0x7FFFFFFFL) return fail(QMV_EINVAL, "qmv_moe_down: n_tokens*top_k overflows");
    if (n_tokens == 0 || N == 0) return QMV_OK;
    if (!Wv || !G || !ids || !weights || !out) return fail(QMV_EINVAL, "qmv_moe_down: NULL W, G, ids, weights or out");
    if (K == 0)
        return fail(QMV_EUNSUPPORTED, "qmv_moe_down: K=0 (qmv_id_swiglu + qmv_moe_wsum cover empty rows)");
    const size_t row = (size_t)(K / QK) * bb;
    if (ldw_bytes < row) return fail(QMV_EINVAL, "qmv_moe_down: ldw_bytes=%zu < K/32*%d=%zu", ldw_bytes, bb, row);
    if ((size_t)N > SIZE_MAX / ldw_bytes) return fail(QMV_EINVAL, "qmv_moe_down: N*ldw overflows");
    if (expert_stride_bytes < (size_t)N * ldw_bytes)
        return fail(QMV_EINVAL, "qmv_moe_down: expert_stride_bytes=%zu < N*ldw_bytes=%zu", expert_stride_bytes,
                    (size_t)N * ldw_bytes);
    if (ldg < (size_t)2 * K) return fail(QMV_EINVAL, "qmv_moe_down: ldg=%zu < 2K=%d", ldg, 2 * K);
    if (ldo < (size_t)N) return fail(QMV_EINVAL, "qmv_moe_down: ldo=%zu < N=%d", ldo, N);
    if (((uintptr_t)G & 3) || ((uintptr_t)out & 3) || ((uintptr_t)ids & 3) || ((uintptr_t)weights & 3) ||
        ((uintptr_t)expert_scale & 3) || ((uintptr_t)err_flag & 3))
        return fail(QMV_EALIGN, "qmv_moe_down: G, out, ids, weights, expert_scale and err_flag must be 4-byte aligned");
    if (K % 64 || ((uintptr_t)Wv & 3) || (ldw_bytes & 3) || (expert_stride_bytes & 3))
        return fail(QMV_EUNSUPPORTED,
                    "qmv_moe_down: needs K %% 64 == 0 and 4-byte aligned W, ldw_bytes and expert_stride_bytes "
                    "(qmv_id_swiglu + qmv_moe_wsum cover the rest)");
    if (top_k > MD_MAX_TOPK || (size_t)top_k * xs_bytes(K) > MD_LDS_MAX)
        return fail(QMV_EUNSUPPORTED,
                    "qmv_moe_down: top_k=%d rows of K=%d do not fit the staging limit (top_k <= %d, top_k*K <= %d); "
                    "qmv_id_swiglu + qmv_moe_wsum cover the rest",
                    top_k, K, MD_MAX_TOPK, (int)(MD_LDS_MAX / xs_bytes(64)) * 64);
    const size_t P = (size_t)n_tokens * top_k;
    const size_t obytes = ((size_t)(n_tokens - 1) * ldo + N) * 4;
    const size_t wbytes = (size_t)(n_experts - 1) * expert_stride_bytes + (size_t)(N - 1) * ldw_bytes + row;
    const size_t gbytes = ((P - 1) * ldg + 2 * (size_t)K) * 4;
    if (overlaps(out, obytes, Wv, wbytes) || overlaps(out, obytes, G, gbytes) || overlaps(out, obytes, ids, P * 4) ||
        overlaps(out, obytes, weights, P * 4) ||
        overlaps(out, obytes, expert_scale, expert_scale ? (size_t)n_experts * 4 : 0) ||
        overlaps(out, obytes, err_flag, err_flag ? 4 : 0))
        return fail(QMV_EINVAL, "qmv_moe_down: out overlaps another argument");
    const uint8_t* W = (const uint8_t*)Wv;
    hipStream_t st = (hipStream_t)stream;
    return qtype == QMV_Q4_0 ? launch_moe_down<QMV_Q4_0>(W, expert_stride_bytes, ldw_bytes, n_experts, G, ldg, ids,
                                                         weights, n_tokens, top_k, out, ldo, N, K, expert_scale,
                                                         err_flag, st)
                             : launch_moe_down<QMV_Q8_0>(W, expert_stride_bytes, ldw_bytes, n_experts, G, ldg, ids,
                                                         weights, n_tokens, top_k, out, ldo, N, K, expert_scale,
                                                         err_flag, st);
}

int qmv_batch(int qtype, const qmv_problem* problems, int n_problems, void* stream) {
    const bool kq = qtype == QMV_Q5_K || qtype == QMV_Q6_K;
    if (qtype != QMV_Q4_0 && qtype != QMV_Q8_0 && !kq)
        return fail(QMV_EUNSUPPORTED, "qmv_batch: qtype %d not supported", qtype);
    if (n_problems < 0 || n_problems > QMV_MAX_BATCH)
        return fail(QMV_EINVAL, "qmv_batch: n_problems=%d outside 0..%d", n_problems, QMV_MAX_BATCH);
    if (n_problems == 0) return QMV_OK;
    if (!problems) return fail(QMV_EINVAL, "qmv_batch: problems is NULL");
    // bytes per block of qk weights
    const int qk = kq ? 256 : QK;
    const int bb = qtype == QMV_Q5_K ? Q5_SB_BYTES : qtype == QMV_Q6_K ? Q6_SB_BYTES : block_bytes(qtype);
    size_t wb[QMV_MAX_BATCH], xb[QMV_MAX_BATCH], yb[QMV_MAX_BATCH];
    for (int i = 0; i < n_problems; ++i) {
        const qmv_problem& p = problems[i];
        if (p.N < 0) return fail(QMV_EINVAL, "qmv_batch: problem %d: N=%d < 0", i, p.N);
        if (p.K < 0 || p.K % qk) return fail(QMV_EINVAL, "qmv_batch: problem %d: K=%d is not a non-negative multiple of %d", i, p.K, qk);
        if (kq && p.K > KMAX_Q6) return fail(QMV_EUNSUPPORTED, "qmv_batch: problem %d: K=%d exceeds %d", i, p.K, KMAX_Q6);
        const size_t row = (size_t)(p.K / qk) * bb;
        if (p.N > 0 && !p.y) return fail(QMV_EINVAL, "qmv_batch: problem %d: y is NULL", i);
        if (p.N > 0 && p.K > 0 && (!p.W || !p.x)) return fail(QMV_EINVAL, "qmv_batch: problem %d: W or x is NULL", i);
        if (p.ldw_bytes < row) return fail(QMV_EINVAL, "qmv_batch: problem %d: ldw_bytes=%zu < K/%d*%d=%zu", i, p.ldw_bytes, qk, bb, row);
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
    if (kq) {
        // Super-block types: problems that share x and K (K > 0) in one
        // launch of k_q6kc; any others, and K = 0, one call each.
        M1Prob sh[QMV_MAX_BATCH];
        int ns = 0;
        const float* x0 = nullptr;
        int K0 = -1;
        for (int i = 0; i < n_problems; ++i)
            if (problems[i].N > 0 && problems[i].K > 0) {
                x0 = problems[i].x;
                K0 = problems[i].K;
                break;
            }
        for (int i = 0; i < n_problems; ++i) {
            const qmv_problem& p = problems[i];
            if (p.N == 0) continue;
            const uint8_t* W = (const uint8_t*)p.W;
            if (p.K > 0 && p.x == x0 && p.K == K0) {
                M1Prob& q = sh[ns++];
                q.W = W;
                q.x = p.x;
                q.y = p.y;
                q.ldw = p.ldw_bytes;
                q.N = p.N;
                q.K = p.K;
                continue;
            }
            int rc;
            if (p.K == 0)
                rc = launch_generic<QMV_Q4_0>(W, p.ldw_bytes, p.x, 0, p.y, p.N, 1, p.N, 0, st);
            else
                rc = qtype == QMV_Q5_K ? launch_q6k<FmtQ5K>(W, p.ldw_bytes, p.x, p.K, p.y, p.N, 1, p.N, p.K, 0, 0, st)
                                       : launch_q6k<FmtQ6K>(W, p.ldw_bytes, p.x, p.K, p.y, p.N, 1, p.N, p.K, 0, 0, st);
            if (rc) return rc;
        }
        if (ns == 0) return QMV_OK;
        return qtype == QMV_Q5_K ? launch_q6kc<FmtQ5K>(sh, ns, st) : launch_q6kc<FmtQ6K>(sh, ns, st);
    }
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

int qmv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (bytes == 0) return QMV_OK;
    if (!src || !sink) return fail(QMV_EINVAL, "qmv_stream_read: NULL src or sink");
    if (((uintptr_t)src & 15) || (bytes & 15) || ((uintptr_t)sink & 3))
        return fail(QMV_EALIGN, "qmv_stream_read: src and bytes must be 16-byte aligned, sink 4-byte aligned");
    const size_t n16 = bytes / 16, chunks = n16 / 2048;
    size_t grid = (size_t)num_cus() * 8;
    grid = grid < chunks ? grid : (chunks ? chunks : 1);
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n16,
                       sink);
    return check_launch("qmv_stream_read");
}



}  // extern "C"
