// fa2_common.h -- device and host helpers shared by the forward
// (fa2_fwd.hip) and backward (fa2_bwd.hip) attention kernels for gfx950.
// Everything here sits in an anonymous namespace, so each translation unit
// gets its own internal copy.
#ifndef FA2_COMMON_H_
#define FA2_COMMON_H_

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "fa2.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Buffer resource over `bytes` bytes at `base` (raw, no stride, dword data
// format): loads past the end return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Workgroup barrier for LDS hand-offs between waves.  It waits for this
// wave's own LDS operations only; __syncthreads would also drain every
// outstanding global->LDS copy (its release fence covers global memory), which
// forces copies issued for a later tile to land early.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt untouched
    __asm__ volatile("s_barrier" ::: "memory");
}

// Copy of one BN-row K or V tile (rows kt*BN ...) of the head at `head` into
// LDS by buffer loads, 16 bytes per lane per load.  `off` holds this lane's
// kLoads byte offsets inside a tile
// (row * row_bytes + swizzled chunk), fixed for the whole kernel; the tile
// offset is a scalar and the LDS destination of a load is wave-uniform
// (M0 + 16 * lane), so outside the last tile a copy costs no vector ALU work.
// Rows past N re-read row N-1 (finite data; their scores are masked).
template <int kLoads, int kRowBytes, int BN>
__device__ __forceinline__ void copy_tile_to_lds(const void* head, const uint32_t* off,
                                                 int wave_u, int kt, int N, char* dst) {
    // the buffer covers one head's K (V): the range check backs up the clamp
    const auto rsrc = make_rsrc(head, N * kRowBytes);
    // (the tile index is the same in every lane; saying so keeps the tile
    // offset in a scalar register where the compiler cannot prove it, which
    // would otherwise turn each load into a loop over distinct offsets)
    const int kbase = __builtin_amdgcn_readfirstlane(kt) * BN;
    const int soff = kbase * kRowBytes;
    char* wdst = dst + wave_u * kLoads * 1024;
    if (kbase + BN <= N) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(wdst + i * 1024),
                                                     16, off[i], soff, 0, 0);
    } else {
        const uint32_t last = (uint32_t)(N - 1 - kbase);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const uint32_t o = min(off[i] / kRowBytes, last) * kRowBytes + off[i] % kRowBytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(wdst + i * 1024),
                                                     16, o, soff, 0, 0);
        }
    }
}

// Row of the 32x32 MFMA accumulator held in register r (0..15) by a lane in
// half h (= lane / 32); the column is lane % 32.
__device__ __forceinline__ constexpr int acc_row(int r, int h) {
    return 8 * (r >> 2) + 4 * h + (r & 3);
}

__device__ __forceinline__ float xchg_half(float x) {
    // value of the lane in the other 32-lane half (same accumulator column)
    return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The 16-bit input types share every kernel; they differ only in the MFMA
// opcode, the conversion that rounds P and O (to nearest even in both), the
// packed sum of two rounded weights and the range a weight may take.
template <typename E>
struct Half;
template <>
struct Half<__bf16> {
    using v8 = bf16x8;
    using v2 = bf16x2;
    // largest sum of softmax weights a lane may accept without moving the
    // running max: every weight is then below it, and bf16 has fp32's range
    static constexpr float kWeightSumCap = 0x1p32f;
    static __device__ __forceinline__ floatx16 mfma(v8 a, v8 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float sum2(v2 p, float acc) {  // acc + p.x + p.y
        const v2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
    }
    static __device__ __forceinline__ float dot2(v2 a, v2 b, float acc) {  // acc + a.x b.x + a.y b.y
        return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
    }
};
template <>
struct Half<_Float16> {
    using v8 = f16x8;
    using v2 = f16x2;
    static constexpr float kWeightSumCap = 0x1p15f;  // fp16 ends at 65504
    static __device__ __forceinline__ floatx16 mfma(v8 a, v8 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float sum2(v2 p, float acc) {
        const v2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(p, one, acc, false);
    }
    static __device__ __forceinline__ float dot2(v2 a, v2 b, float acc) {
        return __builtin_amdgcn_fdot2(a, b, acc, false);
    }
};

// Two floats rounded to nearest even and packed (one v_cvt_pk_*_f32).
template <typename E>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const typename Half<E>::v2 v = {(E)lo, (E)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Which keys a query row sees.
constexpr int kMaskNone = 0;    // all of them
constexpr int kMaskCausal = 1;  // key j visible to query i iff j <= i (top-left)
constexpr int kMaskLocal = 2;   // sliding window i - wl <= j <= i + wr, either side unbounded when -1
                                // (causal with a window is wr = 0)

// First and last key that query row i of a sequence of N keys sees (lo > hi:
// none), for window sides wl, wr.
template <int MASK>
__device__ __forceinline__ int key_lo(int wl, int i) {
    return (MASK == kMaskLocal && wl >= 0) ? max(0, i - wl) : 0;
}
template <int MASK>
__device__ __forceinline__ int key_hi(int wr, int i, int N) {
    int hi = N - 1;
    if (MASK == kMaskCausal) hi = min(hi, i);
    if (MASK == kMaskLocal && wr >= 0) hi = min(hi, i + wr);
    return hi;
}
// First and last query row of a sequence of M rows that sees key j (the
// same relation read the other way).
template <int MASK>
__device__ __forceinline__ int query_lo(int wr, int j) {
    if (MASK == kMaskCausal) return j;
    return (MASK == kMaskLocal && wr >= 0) ? max(0, j - wr) : 0;
}
template <int MASK>
__device__ __forceinline__ int query_hi(int wl, int j, int M) {
    return (MASK == kMaskLocal && wl >= 0) ? min(M - 1, j + wl) : M - 1;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------
bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Status of a kernel launch: the runtime finding no device, or no code object
// for the current device (this library holds gfx950 code only), is
// FA2_ERR_NO_DEVICE; any other refusal is FA2_ERR_LAUNCH.
int launch_status(hipError_t e) {
    switch (e) {
        case hipSuccess: return FA2_OK;
        case hipErrorNoDevice:
        case hipErrorInvalidDevice:
        case hipErrorNoBinaryForGpu:
        case hipErrorInvalidDeviceFunction:
        case hipErrorInsufficientDriver: return FA2_ERR_NO_DEVICE;
        default: return FA2_ERR_LAUNCH;
    }
}

// The problem as the kernels see it.  Without a causal mask, the G query
// heads that share a K/V head are consecutive in q, o and lse, so their rows
// form one contiguous sequence of G*M rows against that K/V head: running
// them as one head of G*M rows reads each K/V tile once per group instead of
// once per query head, and fills the query tiles when M is small (decoding).
// The causal mask depends on the row index within a head, so causal problems
// keep their heads apart.
struct KernelShape {
    int64_t BH, H, G, M;
};
KernelShape kernel_shape(int64_t B, int64_t H, int64_t Hk, int64_t M, int causal) {
    const int64_t G = H > 0 ? H / Hk : 1;
    if (!causal && G > 1) return {B * Hk, Hk, 1, M * G};
    return {B * H, H, G, M};
}

// Window sides as the kernels take them: causal is a right bound of 0; a
// side that reaches past every row (left >= M, right >= N) is unbounded (-1),
// which also keeps i - wl and i + wr inside int.  The mask kind follows.
int normalise_window(int64_t& wl, int64_t& wr, int causal, int64_t M, int64_t N) {
    if (causal) wr = 0;
    if (wl >= M) wl = -1;
    if (wr >= N) wr = -1;
    if (wl < 0 && wr < 0) return kMaskNone;
    if (wl < 0 && wr == 0) return kMaskCausal;
    return kMaskLocal;
}

}  // namespace

#endif  // FA2_COMMON_H_
