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
        u32x4 t = __builtin_nontemporal_load(v + i);
        r[4 * i + 0] = t.x;
        r[4 * i + 1] = t.y;
        r[4 * i + 2] = t.z;
        r[4 * i + 3] = t.w;
    }
    if constexpr (DW % 4) {
        r[DW - 1] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p) + (DW - 1));
    }
}

// LDS layout of the staged activation row: 64 floats per pair of blocks,
// padded to 68 so that lanes reading different pairs use different banks.
constexpr int XS_PAIR = 68;

__host__ __device__ constexpr size_t xs_bytes(int K) { return (size_t)(K / 64) * XS_PAIR * sizeof(float); }

__device__ __forceinline__ void stage_x(float* xs, const float* __restrict__ x, int K) {
    for (int k = threadIdx.x; k < K; k += blockDim.x) xs[(k >> 6) * XS_PAIR + (k & 63)] = x[k];
}

template <int LPR>
__device__ __forceinline__ float lane_group_sum(float v) {
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, LPR);
    return v;
}

// Rows [row0, row0 + RPT) of one M = 1 product, for a lane at position j of
// its LPR-lane group. Weights at W (row stride ldw), activations in xs (LDS).
// Returns the lane's partial sums; the caller reduces over the lane group.
template <int QT, int LPR, int RPT>
__device__ __forceinline__ void m1_rows(const uint8_t* __restrict__ W, size_t ldw, const float* xs, int P,
                                        long row0, int N, int j, float* tot) {
    using T = PairTraits<QT>;
    constexpr int PB = T::DW * 4;
    const uint8_t* wp[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        long rr = row0 + r < N ? row0 + r : N - 1;
        wp[r] = W + rr * ldw;
        tot[r] = 0.f;
    }
    for (int p = j; p < P; p += LPR) {
        uint32_t buf[RPT][T::DW];
#pragma unroll
        for (int r = 0; r < RPT; ++r) load_pair<T::DW>(wp[r] + (size_t)p * PB, buf[r]);
        const float4* xv = reinterpret_cast<const float4*>(xs + p * XS_PAIR);
#pragma unroll
        for (int r = 0; r < RPT; ++r) tot[r] += T::dot(buf[r], xv);
    }
}

// ---------------------------------------------------------------------------
// M = 1 dense kernel (fast path). Requires K % 64 == 0, W and ldw 4-aligned.
// ---------------------------------------------------------------------------
template <int QT, int LPR, int RPT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_m1(const uint8_t* __restrict__ W, size_t ldw,
                                                   const float* __restrict__ x, float* __restrict__ y, int N, int K) {
    extern __shared__ __align__(16) float xs[];
    stage_x(xs, x, K);
    __syncthreads();
    constexpr int GROUPS = 64 / LPR;
    constexpr int ROWS_PER_WG = GROUPS * RPT * WAVES;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPR, j = lane % LPR;
    const int P = K >> 6;
    for (long tile = blockIdx.x; tile * ROWS_PER_WG < N; tile += gridDim.x) {
        const long row0 = tile * ROWS_PER_WG + (long)(wave * GROUPS + g) * RPT;
        float tot[RPT];
        m1_rows<QT, LPR, RPT>(W, ldw, xs, P, row0, N, j, tot);
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            float s = lane_group_sum<LPR>(tot[r]);
            if (j == 0 && row0 + r < N) y[row0 + r] = s * PairTraits<QT>::OUT_SCALE;
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
    const int lane = tid & 63, wave = tid >> 6;

    if (count == 1 && fast) {
        const int t = p / top_k;
        stage_x(xs, X + (size_t)t * ldx, K);
        __syncthreads();
        const int g = lane / LPR, j = lane % LPR;
        const long row0 = tile_row0 + (long)(wave * GROUPS + g) * RPT;
        float tot[RPT];
        m1_rows<QT, LPR, RPT>(We, ldw, xs, K >> 6, row0, N, j, tot);
        const float sc = (escale ? escale[e] : 1.f) * PairTraits<QT>::OUT_SCALE;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            float s = lane_group_sum<LPR>(tot[r]);
            if (j == 0 && row0 + r < N) Y[(size_t)p * ldy + row0 + r] = s * sc;
        }
        return;
    }
    // General case: one wave per row, up to 16 pairs per pass.
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

struct M1Shape {
    int lpr, rpt;
};

// Lanes per row: the largest power of two (<= 64) whose lane utilisation
// P / (LPR * ceil(P / LPR)) is within 5% of the best one, so long rows keep
// a full wave on one row and short rows still use every lane.
int pick_lpr(int P) {
    double best = 0;
    int cands[] = {64, 32, 16, 8, 4};
    double eff[5];
    for (int i = 0; i < 5; ++i) {
        int l = cands[i];
        eff[i] = (double)P / ((double)l * ((P + l - 1) / l));
        if (eff[i] > best) best = eff[i];
    }
    for (int i = 0; i < 5; ++i)
        if (eff[i] >= best * 0.95) return cands[i];
    return 4;
}

M1Shape pick_m1(int N, int K) {
    M1Shape s;
    s.lpr = pick_lpr(K / 64);
    s.rpt = (N >= 4096) ? 2 : 1;
    return s;
}

template <int QT, int LPR, int RPT>
int launch_m1_t(const uint8_t* W, size_t ldw, const float* X, float* Y, int N, int K, hipStream_t st) {
    constexpr int WAVES = 4;
    constexpr int ROWS_PER_WG = (64 / LPR) * RPT * WAVES;
    const long tiles = ((long)N + ROWS_PER_WG - 1) / ROWS_PER_WG;
    const int grid = (int)(tiles < 65535 ? tiles : 65535);
    hipLaunchKernelGGL((k_m1<QT, LPR, RPT, WAVES>), dim3(grid), dim3(WAVES * 64), xs_bytes(K), st, W, ldw, X, Y,
                       N, K);
    return check_launch("qmv m1 kernel");
}

template <int QT>
int launch_m1(const uint8_t* W, size_t ldw, const float* X, float* Y, int N, int K, hipStream_t st) {
    M1Shape s = pick_m1(N, K);
#define QMV_M1_CASE(L, R) \
    if (s.lpr == L && s.rpt == R) return launch_m1_t<QT, L, R>(W, ldw, X, Y, N, K, st);
    QMV_M1_CASE(64, 1) QMV_M1_CASE(64, 2) QMV_M1_CASE(32, 1) QMV_M1_CASE(32, 2) QMV_M1_CASE(16, 1)
    QMV_M1_CASE(16, 2) QMV_M1_CASE(8, 1) QMV_M1_CASE(8, 2) QMV_M1_CASE(4, 1) QMV_M1_CASE(4, 2)
#undef QMV_M1_CASE
    return fail(QMV_EINVAL, "internal: no m1 kernel for lpr=%d rpt=%d", s.lpr, s.rpt);
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

const char* qmv_last_error(void) { return g_err; }

#ifdef QMV_PROBE
// Tuning entry, built only into a separate probe library: run the M = 1
// kernel with an explicit lanes-per-row / rows-per-lane choice.
int qmv_probe_m1(int qtype, int lpr, int rpt, const void* W, size_t ldw, const float* X, float* Y, int N, int K,
                 void* stream) {
    hipStream_t st = (hipStream_t)stream;
    const uint8_t* w = (const uint8_t*)W;
#define QMV_P(QT, L, R) \
    if (qtype == QT && lpr == L && rpt == R) return launch_m1_t<QT, L, R>(w, ldw, X, Y, N, K, st);
#define QMV_PQ(QT) QMV_P(QT, 64, 1) QMV_P(QT, 64, 2) QMV_P(QT, 64, 4) QMV_P(QT, 32, 1) QMV_P(QT, 32, 2) \
    QMV_P(QT, 32, 4) QMV_P(QT, 16, 1) QMV_P(QT, 16, 2) QMV_P(QT, 16, 4) QMV_P(QT, 8, 1) QMV_P(QT, 8, 2) QMV_P(QT, 4, 1)
    QMV_PQ(QMV_Q4_0) QMV_PQ(QMV_Q8_0)
#undef QMV_PQ
#undef QMV_P
    return fail(QMV_EINVAL, "probe: no variant");
}
#endif

}  // extern "C"
