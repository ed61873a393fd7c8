// qmv_internal.h — pieces shared by the library's translation units (not part
// of the C ABI): error reporting, device queries, and the device helpers that
// read GGML blocks and move operands between lanes.
#ifndef QMV_INTERNAL_H
#define QMV_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "qmv.h"

#define QMV_HIDDEN __attribute__((visibility("hidden")))

namespace qmvi {

// ---------------------------------------------------------------------------
// Host side (defined in qmv.hip)
// ---------------------------------------------------------------------------
// Sets the thread-local message read by qmv_last_error() and returns code.
QMV_HIDDEN int fail(int code, const char* fmt, ...);
// QMV_EHIP with a message if the last launch failed, QMV_OK otherwise.
QMV_HIDDEN int check_launch(const char* what);
// Compute units of the current device.
QMV_HIDDEN int num_cus();

// Matrix-core products (qmv_mq.hip), any number of activation rows in blocks
// of 16. Requirements, checked by the caller: qtype Q4_0 or Q8_0, K > 0 and
// K % 64 == 0, W and ldw 4-byte aligned, X and Y 4-byte aligned, M >= 1.
// ws / ws_bytes: a caller workspace the call may use for K-segment partial
// sums (NULL / 0: none; the call then needs no memory beyond X, W and Y).
// The launch shape follows from M, N, K and the workspace given (ws_bytes of
// it at ws; none: ws = nullptr).
QMV_HIDDEN int launch_mq(int qtype, const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy,
                         int M, int N, int K, void* ws, size_t ws_bytes, hipStream_t st);
// Workspace bytes launch_mq would use for M, N, K given unlimited room (0 if
// it would not split K).
QMV_HIDDEN size_t mq_ws_bytes(int M, int N, int K);
// Tiled matrix-core product for many activation rows (qmv_mq.hip): tiles of
// 64 x 256 outputs, each weight decoded once per tile. Requirements, checked
// by the caller: qtype Q4_0 or Q8_0, K > 0 and K % 64 == 0, W and ldw 4-byte
// aligned, ldw < 2^32, X 16-byte aligned, ldx % 4 == 0, Y 4-byte aligned.
QMV_HIDDEN int launch_gemm(int qtype, const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy,
                           int M, int N, int K, hipStream_t st);
// Expert-indexed product on the matrix cores (qmv_mq.hip), Q4_0 or Q8_0.
// Requirements, checked by the caller: K >= 256 and K % 64 == 0, at most 1024
// pairs and 1024 experts, W, ldw and es 4-byte aligned, ldw < 2^32, X
// 16-byte aligned, ldx % 4 == 0, the launch's X rows below 2 GiB.
QMV_HIDDEN int launch_idq(int qtype, const uint8_t* W, size_t es, size_t ldw, int E, const float* X, size_t ldx,
                          const uint32_t* ids, int n_pairs, int top_k, float* Y, size_t ldy, int N, int K,
                          const float* sc, int* err, hipStream_t st);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The binary16 in the low / high half of w, as fp32 (exact, subnormals kept).
__device__ __forceinline__ float half_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// (code - 8) / 16 for the low nibble of byte B of w, where w holds code
// bytes XORed with 0x88 (v_cvt_off_f32_i4 reads bits [3:0] as a signed 4-bit
// value and divides by 16; code ^ 8 read that way is code - 8). The byte is
// selected with a shift and mask that the compiler folds into the
// instruction's SDWA operand select, so no separate shift is issued.
template <int B>
__device__ __forceinline__ float nib(uint32_t w) {
    if constexpr (B == 0) return __builtin_amdgcn_cvt_off_f32_i4((int)w);
    else if constexpr (B == 3) return __builtin_amdgcn_cvt_off_f32_i4((int)(w >> 24));
    else return __builtin_amdgcn_cvt_off_f32_i4((int)((w >> (8 * B)) & 0xFFu));
}

// w with each byte's high nibble moved into its low nibble, for nib<B>. A
// rotation rather than a shift, so that the compiler cannot prove the other
// bits of each byte zero and narrow nib's byte mask, which would stop it from
// folding the byte select into the convert.
__device__ __forceinline__ uint32_t hi_nibbles(uint32_t w) { return (w >> 4) | (w << 28); }

// DW dwords from a 4-byte aligned address, with 16-byte vector loads.
template <int DW>
__device__ __forceinline__ void load_pair(const uint8_t* p, uint32_t* r) {
    const u32x4* v = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < DW / 4; ++i) {
        const u32x4 t = v[i];
        r[4 * i + 0] = t.x;
        r[4 * i + 1] = t.y;
        r[4 * i + 2] = t.z;
        r[4 * i + 3] = t.w;
    }
    if constexpr (DW % 4) {
#pragma unroll
        for (int i = DW & ~3; i < DW; ++i) r[i] = reinterpret_cast<const uint32_t*>(p)[i];
    }
}

// Compile-time unrolled loop helper.
template <int I, int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        unroll<I + 1, N>(f);
    }
}

// An empty volatile asm that reads and rewrites the N registers of b and
// clobbers memory. Placed after the next step's loads are issued, it keeps
// the decode of b below them: otherwise the compiler may hoist part of the
// decode above the issue, and its wait for b's loads then holds back the
// next loads, leaving one step in flight instead of two.
template <int N>
__device__ __forceinline__ void pin_regs(uint32_t* b) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(b[i])::"memory");
}

// Load instructions load_pair<DW> issues.
template <int DW>
constexpr int pair_loads() { return DW / 4 + DW % 4; }

// s_waitcnt vmcnt(N): wait until at most N vector memory operations of this
// wave are outstanding. Also tells the compiler's wait bookkeeping that the
// older ones are done, which it cannot infer after loads and LDS stores made
// conditional per lane (it would otherwise wait for them again later, at the
// first reuse of their registers, behind loads issued since).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 4 x 4 transpose across the four 16-lane rows of a wave: on entry lane row
// R holds v[c] = element (R, c); on exit it holds v[c] = element (c, R).
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

// Workgroup barrier over LDS only: waits for this thread's LDS operations but
// not for its outstanding global loads (__syncthreads waits for those too,
// which would drain the weight loads already in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


// Expert grouping shared by the expert-indexed kernels that serve many pairs.
constexpr int IDP_MAX_EXPERTS = 1024;  // experts the LDS tables index
constexpr int IDP_MAX_PAIRS = 1024;    // pairs one launch groups

// Groups the launch's pairs by expert in LDS (all NT threads of the
// workgroup take part): the distinct experts u = 0 .. U-1 in order of first
// appearance (s_uexp[u]), the pairs of u at s_plist[s_ustart[u] ..
// s_ustart[u + 1]) (in no fixed order: they are filled with atomics, and no
// result depends on it), s_map[e] = u. A pair whose id is outside
// [0, n_experts) gets a NaN output row and sets *err_flag (those rows spread
// over the workgroups). Returns U.
template <int NT>
__device__ __forceinline__ int group_by_expert(const uint32_t* __restrict__ ids, int n_pairs, int n_experts,
                                               int* s_map, int* s_uexp, int* s_ustart, int* s_cnt, int* s_plist,
                                               int* s_U, float* __restrict__ Y, size_t ldy, int N,
                                               int* __restrict__ err_flag) {
    constexpr int QPT = IDP_MAX_PAIRS / NT;  // ids per thread
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t myid[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        const int q = tid + k * NT;
        myid[k] = q < n_pairs ? ids[q] : 0xFFFFFFFFu;
    }
    for (int e = tid; e < n_experts; e += NT) s_map[e] = 0x7FFFFFFF;
    for (int u = tid; u < IDP_MAX_PAIRS; u += NT) s_cnt[u] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < QPT; ++k)
        if (myid[k] < (uint32_t)n_experts) atomicMin(&s_map[myid[k]], tid + k * NT);
    __syncthreads();
    if (wave == 0) {  // distinct experts in order of first appearance
        int base = 0;
        for (int q0 = 0; q0 < n_pairs; q0 += 64) {
            const int q = q0 + lane;
            const uint32_t e = q < n_pairs ? ids[q] : 0xFFFFFFFFu;
            const bool first = e < (uint32_t)n_experts && s_map[e] == q;
            const uint64_t m = __ballot(first);
            if (first) s_uexp[base + __popcll(m & ((1ull << lane) - 1ull))] = (int)e;
            base += __popcll(m);
        }
        if (lane == 0) *s_U = base;
    }
    __syncthreads();
    const int U = *s_U;
    for (int u = tid; u < U; u += NT) s_map[s_uexp[u]] = u;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < QPT; ++k)
        if (myid[k] < (uint32_t)n_experts) atomicAdd(&s_cnt[s_map[myid[k]]], 1);
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the counts; the counts become cursors
        int base = 0;
        for (int u0 = 0; u0 < U; u0 += 64) {
            const int u = u0 + lane;
            const int c = u < U ? s_cnt[u] : 0;
            int incl = c;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o, 64);
                if (lane >= o) incl += t;
            }
            if (u < U) {
                s_ustart[u] = base + incl - c;
                s_cnt[u] = base + incl - c;
            }
            base += __shfl(incl, 63, 64);
        }
        if (lane == 0) s_ustart[U] = base;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < QPT; ++k)
        if (myid[k] < (uint32_t)n_experts) s_plist[atomicAdd(&s_cnt[s_map[myid[k]]], 1)] = tid + k * NT;
    // pairs with an id out of range: NaN rows, spread over the workgroups
    for (int q = blockIdx.x; q < n_pairs; q += gridDim.x) {
        if (ids[q] >= (uint32_t)n_experts) {
            for (int n = tid; n < N; n += NT) Y[(size_t)q * ldy + n] = __builtin_nanf("");
            if (tid == 0 && err_flag) *err_flag = 1;
        }
    }
    __syncthreads();

    return U;
}

}  // namespace qmvi

#endif
