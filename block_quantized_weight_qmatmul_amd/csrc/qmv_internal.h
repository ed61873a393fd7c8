// qmv_internal.h — pieces shared by the library's translation units (not part
// of the C ABI): error reporting, device queries, and the device helpers that
// read GGML blocks and move operands between lanes.
#ifndef QMV_INTERNAL_H
#define QMV_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
// waves = 0 picks the launch shape; otherwise waves, ks and S force it
// (tuning).
QMV_HIDDEN int launch_mq(int qtype, const uint8_t* W, size_t ldw, const float* X, size_t ldx, float* Y, size_t ldy,
                         int M, int N, int K, void* ws, size_t ws_bytes, int waves, int ks, int S, hipStream_t st);
// Workspace bytes launch_mq would use for M, N, K given unlimited room (0 if
// it would not split K).
QMV_HIDDEN size_t mq_ws_bytes(int M, int N, int K);

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

}  // namespace qmvi

#endif
