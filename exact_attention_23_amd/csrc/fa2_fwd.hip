// fa2_fwd.hip -- exact attention forward pass (FlashAttention-2 schedule) for
// AMD CDNA4 / gfx950, behind the C ABI declared in include/fa2.h.
//
// What is computed: O = softmax(scale * Q K^T) V per (batch, head), optionally
// causal (key j visible to query i iff j <= i), plus L = m + log(l), the
// natural-log logsumexp of each query row's scaled scores.  The schedule is the
// FlashAttention-2 forward described on the pages:
//  * one workgroup per (query tile, batch*head), the K/V loop inside it
//    ("Writing FlashAttention 2 in Triton", Step 1; "From FlashAttention to
//    FlashAttention 2", section "2. Swapping the Loop Order");
//  * the online-softmax recurrence with running max m, running sum l and an
//    unnormalised O, all fp32, rescaled by exp(m_old - m_new) on each K/V tile
//    ("FlashAttention-2 from PyTorch to Triton", the tile loop and the
//    accumulator discussion; "Writing FlashAttention 2 in Triton", Step 4);
//  * one division by l at the end ("Writing FlashAttention 2 in Triton",
//    Step 5; "From FlashAttention to FlashAttention 2", section "1. Reducing
//    Non-Matmul FLOPs");
//  * work split across waves only along query rows, so no wave needs another
//    wave's scores ("From FlashAttention to FlashAttention 2", section "3.
//    Better Work Partitioning Between Warps");
//  * exp2 with scale*log2(e) folded into one FMA ("From FlashAttention to
//    FlashAttention 2", section "Layer 6: The Online Softmax Implementation");
//  * causal tile skipping at the diagonal and masking only on boundary tiles
//    ("Writing FlashAttention 2 in Triton", Step 4; "FlashAttention-2 from
//    PyTorch to Triton", items 2 and 6 of the list of known slowness);
//  * keys past N masked rather than scored as zero ("FlashAttention-2 from
//    PyTorch to Triton", the second fix of its test harness section).
//
// gfx950 mapping (our own design, not the pages' CUDA/Triton tiling):
//  * The score tile is computed transposed, S^T = K Q^T, and the output as
//    O^T += V^T P^T, on 32x32 MFMA tiles.  In the 32x32 accumulator layout
//    lane l owns column l%32, so every lane owns ONE query row: the row max and
//    row sum are in-lane over 16 registers per 32-key block plus one exchange
//    with lane l^32 (which owns the other 16 keys of the same rows).  The
//    per-row rescale factor alpha lives in the same lane as the O^T column it
//    scales, so no cross-lane traffic is needed for the rescale either.
//  * P leaves the S^T accumulator already in the B-operand layout of the PV
//    MFMA (lane = query, 8 keys per lane).  The A operand, V^T, is read from
//    an LDS copy of V stored transposed ([d][key]) with bits 2 and 3 of the key
//    index swapped, which makes the 8 keys a lane needs contiguous: one 16-byte
//    LDS read per MFMA operand.
//  * K and V^T tiles are double-buffered in LDS with padded rows (bank-conflict
//    free 16-byte reads; conflict-free transposing 4-byte writes); the next
//    tile's global loads are issued before the current tile's MFMAs.
//  * Q stays in VGPRs for the whole K/V loop; O^T, m, l stay in registers.
//  * Causal grids launch the heaviest query tiles first; batch*head is the
//    fastest-varying grid index so that all tiles of one head land on the same
//    XCD (workgroups are dealt to the 8 XCDs round-robin).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "fa2.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;

// Row of the 32x32 MFMA accumulator held in register r (0..15) by a lane in
// half h (= lane / 32); the column is lane % 32.
__device__ __forceinline__ constexpr int acc_row(int r, int h) {
    return 8 * (r >> 2) + 4 * h + (r & 3);
}

// Position of key `key` (tile-local) in the transposed V tile: bits 2 and 3
// swapped, so that the 8 keys one lane feeds to a PV MFMA are adjacent.
__device__ __forceinline__ constexpr int vperm(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ __forceinline__ float xchg_half(float x) {
    // value of the lane in the other 32-lane half (same accumulator column)
    return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo;  // round to nearest even
    __bf16 b = (__bf16)hi;
    uint16_t ua, ub;
    __builtin_memcpy(&ua, &a, 2);
    __builtin_memcpy(&ub, &b, 2);
    return (uint32_t)ua | ((uint32_t)ub << 16);
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
// D: head dim (64 or 128); BN: keys per K/V tile (multiple of 32);
// NW: waves per workgroup; QB: 32-query blocks per wave.
template <int D, int BN, int NW, int QB>
struct Bf16Traits {
    static constexpr int kThreads = NW * 64;
    static constexpr int kQPW = 32 * QB;          // query rows per wave
    static constexpr int kBM = kQPW * NW;         // query rows per workgroup
    static constexpr int kKB = BN / 32;           // 32-key blocks per tile
    static constexpr int kDB = D / 32;            // 32-wide d blocks of O^T
    static constexpr int kDS = D / 16;            // MFMA k-steps of S^T
    static constexpr int kKStr = D + 8;           // K tile row stride (elements)
    static constexpr int kVStr = BN + 8;          // V^T tile row stride (elements)
    static constexpr int kKElems = BN * kKStr;
    static constexpr int kVElems = D * kVStr;
    static constexpr int kKChunks = BN * D / 8;   // 16-byte chunks per K tile
    static constexpr int kVPairs = (BN / 2) * (D / 8);  // (key pair, 8-d chunk) items
    static constexpr int kKPerThread = kKChunks / kThreads;
    static constexpr int kVPerThread = kVPairs / kThreads;
    static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");
    static_assert(kKChunks % kThreads == 0 && kVPairs % kThreads == 0, "loader split");
    static constexpr size_t kLdsBytes = 2 * (kKElems + kVElems) * sizeof(__bf16);
};

template <int D, int BN, int NW, int QB, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64)
fa2_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                    const __bf16* __restrict__ V, __bf16* __restrict__ O,
                    float* __restrict__ LSE, int BH, int M, int N, int n_qt,
                    float c_log2) {
    using T = Bf16Traits<D, BN, NW, QB>;
    __shared__ __attribute__((aligned(16))) __bf16 sK[2][T::kKElems];
    __shared__ __attribute__((aligned(16))) __bf16 sV[2][T::kVElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // workgroup -> (batch*head, query tile); causal: heaviest tiles first
    const int wg = blockIdx.x;
    const int bh = wg % BH;
    int qt = wg / BH;
    if (CAUSAL) qt = n_qt - 1 - qt;
    const int q0 = qt * T::kBM;
    const int qw0 = q0 + wave * T::kQPW;  // first query row of this wave

    const __bf16* Qh = Q + (int64_t)bh * M * D;
    const __bf16* Kh = K + (int64_t)bh * N * D;
    const __bf16* Vh = V + (int64_t)bh * N * D;

    // K/V tiles covered by this workgroup, and by this wave
    const int kv_end = CAUSAL ? min(N, q0 + T::kBM) : N;
    const int n_kv = (kv_end + BN - 1) / BN;
    int n_kv_wave = n_kv;
    if (CAUSAL) n_kv_wave = min(n_kv, (min(N, qw0 + T::kQPW) + BN - 1) / BN);
    if (qw0 >= M) n_kv_wave = 0;  // the wave holds only rows past M

    // ---- Q fragments: B operand of S^T = K Q^T (lane = query, 8 d values)
    bf16x8 qf[QB][T::kDS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw0 + 32 * qb + l32;
#pragma unroll
        for (int s = 0; s < T::kDS; ++s) {
            if (row < M) {
                qf[qb][s] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)row * D + 16 * s + 8 * h);
            } else {
                qf[qb][s] = bf16x8{};
            }
        }
    }

    // ---- running state (fp32): O^T accumulators, max (log2 units), partial sum
    floatx16 oacc[T::kDB][QB];
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db) oacc[db][qb] = floatx16{};
    }

    // ---- tile loader: global -> registers -> LDS
    u32x4 kreg[T::kKPerThread];
    u32x4 vreg[T::kVPerThread][2];

    auto load_tile = [&](int kt) {
        const int kbase = kt * BN;
#pragma unroll
        for (int i = 0; i < T::kKPerThread; ++i) {
            const int id = tid + i * T::kThreads;
            const int row = id / (D / 8);
            const int c8 = id % (D / 8);
            const int key = kbase + row;
            kreg[i] = key < N ? *reinterpret_cast<const u32x4*>(Kh + (int64_t)key * D + 8 * c8)
                              : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < T::kVPerThread; ++i) {
            const int id = tid + i * T::kThreads;
            const int a2 = id % (BN / 2);
            const int c8 = id / (BN / 2);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int key = kbase + 2 * a2 + j;
                vreg[i][j] = key < N ? *reinterpret_cast<const u32x4*>(Vh + (int64_t)key * D + 8 * c8)
                                     : u32x4{0, 0, 0, 0};
            }
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::kKPerThread; ++i) {
            const int id = tid + i * T::kThreads;
            const int row = id / (D / 8);
            const int c8 = id % (D / 8);
            *reinterpret_cast<u32x4*>(&sK[buf][row * T::kKStr + 8 * c8]) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < T::kVPerThread; ++i) {
            const int id = tid + i * T::kThreads;
            const int a2 = id % (BN / 2);
            const int c8 = id / (BN / 2);
            const int col = vperm(2 * a2);  // keys 2*a2 and 2*a2+1 stay adjacent
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w0 = vreg[i][0][e >> 1];
                const uint32_t w1 = vreg[i][1][e >> 1];
                const uint32_t packed = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                                : ((w0 & 0xffffu) | (w1 << 16));
                *reinterpret_cast<uint32_t*>(&sV[buf][(8 * c8 + e) * T::kVStr + col]) = packed;
            }
        }
    };

    if (n_kv > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int kt = 0; kt < n_kv; ++kt) {
        const int buf = kt & 1;
        const bool has_next = kt + 1 < n_kv;
        if (has_next) load_tile(kt + 1);

        if (kt < n_kv_wave) {
            const __bf16* kt_lds = sK[buf];
            const __bf16* vt_lds = sV[buf];

            // S^T = K Q^T for BN keys x QPW queries
            floatx16 sacc[T::kKB][QB];
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = floatx16{};
#pragma unroll
            for (int s = 0; s < T::kDS; ++s) {
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
                        kt_lds + (32 * kb + l32) * T::kKStr + 16 * s + 8 * h);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][s], sacc[kb][qb], 0, 0, 0);
                }
            }

            // boundary tiles only: keys past N, and (causal) keys after the query
            const int kbase = kt * BN;
            const bool need_mask = (kbase + BN > N) || (CAUSAL && kbase + BN - 1 > qw0);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        const int query = qw0 + 32 * qb + l32;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kbase + 32 * kb + acc_row(r, h);
                            const bool vis = key < N && (!CAUSAL || key <= query);
                            if (!vis) sacc[kb][qb][r] = -INFINITY;
                        }
                    }
            }

            // online softmax (log2 domain); P overwrites S in place
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
                mx = fmaxf(mx, xchg_half(mx));
                const float m_new = fmaxf(m_run[qb], mx * c_log2);
                // a row with no visible key so far keeps exp2 arguments finite
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = fast_exp2(m_run[qb] - m_use);
                m_run[qb] = m_new;
                float lsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = fast_exp2(fmaf(sacc[kb][qb][r], c_log2, -m_use));
                        sacc[kb][qb][r] = p;
                        lsum += p;
                    }
                l_run[qb] = fmaf(l_run[qb], alpha, lsum);
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) oacc[db][qb] *= alpha;
            }

            // O^T += V^T P^T: two 16-key MFMA steps per 32-key block
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb) {
#pragma unroll
                for (int ms = 0; ms < 2; ++ms) {
                    bf16x8 pf[QB];
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                        for (int t = 0; t < 8; ++t) pf[qb][t] = (__bf16)sacc[kb][qb][8 * ms + t];
#pragma unroll
                    for (int db = 0; db < T::kDB; ++db) {
                        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
                            vt_lds + (32 * db + l32) * T::kVStr + 32 * kb + 16 * ms + 8 * h);
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb)
                            oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb], oacc[db][qb], 0, 0, 0);
                    }
                }
            }
        }

        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: one normalisation, L = (m + log2 l) * ln 2, RNE store
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = l_run[qb] + xchg_half(l_run[qb]);
        const int query = qw0 + 32 * qb + l32;
        if (query < M) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            __bf16* orow = O + ((int64_t)bh * M + query) * D;
#pragma unroll
            for (int db = 0; db < T::kDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = 32 * db + 8 * g + 4 * h;
                    uint32_t w[2];
                    w[0] = pack_bf16x2(oacc[db][qb][4 * g + 0] * inv, oacc[db][qb][4 * g + 1] * inv);
                    w[1] = pack_bf16x2(oacc[db][qb][4 * g + 2] * inv, oacc[db][qb][4 * g + 3] * inv);
                    *reinterpret_cast<uint2*>(orow + d) = make_uint2(w[0], w[1]);
                }
            if (h == 0) LSE[(int64_t)bh * M + query] = (m_run[qb] + fast_log2(l_tot)) * kLn2;
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2_f32: true fp32 products, no reduced-precision
// shortcut)
// ---------------------------------------------------------------------------
template <int D, int BN, int NW>
struct F32Traits {
    static constexpr int kThreads = NW * 64;
    static constexpr int kBM = 32 * NW;
    static constexpr int kKB = BN / 32;
    static constexpr int kDB = D / 32;
    static constexpr int kHalfD = D / 2;          // d values per lane half
    static constexpr int kKStr = D + 4;           // floats
    static constexpr int kVStr = D + 8;           // floats
    static constexpr int kKElems = BN * kKStr;
    static constexpr int kVElems = BN * kVStr;
    static constexpr int kChunks = BN * D / 4;    // 16-byte chunks per tile
    static constexpr int kPerThread = kChunks / kThreads;
    static_assert(kChunks % kThreads == 0, "loader split");
    static constexpr size_t kLdsBytes = 2 * (kKElems + kVElems) * sizeof(float);
};

template <int D, int BN, int NW, bool CAUSAL>
__global__ void __launch_bounds__(NW * 64)
fa2_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                   const float* __restrict__ V, float* __restrict__ O,
                   float* __restrict__ LSE, int BH, int M, int N, int n_qt,
                   float c_log2) {
    using T = F32Traits<D, BN, NW>;
    __shared__ __attribute__((aligned(16))) float sK[2][T::kKElems];
    __shared__ __attribute__((aligned(16))) float sV[2][T::kVElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    const int wg = blockIdx.x;
    const int bh = wg % BH;
    int qt = wg / BH;
    if (CAUSAL) qt = n_qt - 1 - qt;
    const int q0 = qt * T::kBM;
    const int qw0 = q0 + wave * 32;

    const float* Qh = Q + (int64_t)bh * M * D;
    const float* Kh = K + (int64_t)bh * N * D;
    const float* Vh = V + (int64_t)bh * N * D;

    const int kv_end = CAUSAL ? min(N, q0 + T::kBM) : N;
    const int n_kv = (kv_end + BN - 1) / BN;
    int n_kv_wave = n_kv;
    if (CAUSAL) n_kv_wave = min(n_kv, (min(N, qw0 + 32) + BN - 1) / BN);
    if (qw0 >= M) n_kv_wave = 0;

    // Q: lane half h holds d in [h*D/2, (h+1)*D/2) of its query row; MFMA step s
    // contracts d = h*D/2 + s in both operands.
    float qf[T::kHalfD];
    {
        const int row = qw0 + l32;
#pragma unroll
        for (int s = 0; s < T::kHalfD; s += 4) {
            floatx4 x = floatx4{0.f, 0.f, 0.f, 0.f};
            if (row < M) x = *reinterpret_cast<const floatx4*>(Qh + (int64_t)row * D + h * T::kHalfD + s);
            qf[s] = x[0]; qf[s + 1] = x[1]; qf[s + 2] = x[2]; qf[s + 3] = x[3];
        }
    }

    floatx16 oacc[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) oacc[db] = floatx16{};
    float m_run = -INFINITY, l_run = 0.f;

    u32x4 kreg[T::kPerThread], vreg[T::kPerThread];
    auto load_tile = [&](int kt) {
        const int kbase = kt * BN;
#pragma unroll
        for (int i = 0; i < T::kPerThread; ++i) {
            const int id = tid + i * T::kThreads;
            const int row = id / (D / 4);
            const int c4 = id % (D / 4);
            const int key = kbase + row;
            const bool ok = key < N;
            kreg[i] = ok ? *reinterpret_cast<const u32x4*>(Kh + (int64_t)key * D + 4 * c4) : u32x4{0, 0, 0, 0};
            vreg[i] = ok ? *reinterpret_cast<const u32x4*>(Vh + (int64_t)key * D + 4 * c4) : u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::kPerThread; ++i) {
            const int id = tid + i * T::kThreads;
            const int row = id / (D / 4);
            const int c4 = id % (D / 4);
            *reinterpret_cast<u32x4*>(&sK[buf][row * T::kKStr + 4 * c4]) = kreg[i];
            *reinterpret_cast<u32x4*>(&sV[buf][row * T::kVStr + 4 * c4]) = vreg[i];
        }
    };

    if (n_kv > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int kt = 0; kt < n_kv; ++kt) {
        const int buf = kt & 1;
        const bool has_next = kt + 1 < n_kv;
        if (has_next) load_tile(kt + 1);

        if (kt < n_kv_wave) {
            const float* kt_lds = sK[buf];
            const float* vt_lds = sV[buf];

            floatx16 sacc[T::kKB];
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb) sacc[kb] = floatx16{};
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb) {
                const float* krow = kt_lds + (32 * kb + l32) * T::kKStr + h * T::kHalfD;
#pragma unroll
                for (int s = 0; s < T::kHalfD; s += 4) {
                    const floatx4 kf = *reinterpret_cast<const floatx4*>(krow + s);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[u], qf[s + u], sacc[kb], 0, 0, 0);
                }
            }

            const int kbase = kt * BN;
            const bool need_mask = (kbase + BN > N) || (CAUSAL && kbase + BN - 1 > qw0);
            if (need_mask) {
                const int query = qw0 + l32;
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + 32 * kb + acc_row(r, h);
                        const bool vis = key < N && (!CAUSAL || key <= query);
                        if (!vis) sacc[kb][r] = -INFINITY;
                    }
            }

            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, xchg_half(mx));
            const float m_new = fmaxf(m_run, mx * c_log2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            m_run = m_new;
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(sacc[kb][r], c_log2, -m_use));
                    sacc[kb][r] = p;
                    lsum += p;
                }
            l_run = fmaf(l_run, alpha, lsum);
#pragma unroll
            for (int db = 0; db < T::kDB; ++db) oacc[db] *= alpha;

            // O^T += V^T P^T: MFMA step r contracts key acc_row(r, h) in each half
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float* vrow = vt_lds + (32 * kb + acc_row(r, h)) * T::kVStr + l32;
#pragma unroll
                    for (int db = 0; db < T::kDB; ++db)
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * db], sacc[kb][r], oacc[db], 0, 0, 0);
                }
        }

        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    const float l_tot = l_run + xchg_half(l_run);
    const int query = qw0 + l32;
    if (query < M) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* orow = O + ((int64_t)bh * M + query) * D;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * db + 8 * g + 4 * h;
                floatx4 x;
                x[0] = oacc[db][4 * g + 0] * inv;
                x[1] = oacc[db][4 * g + 1] * inv;
                x[2] = oacc[db][4 * g + 2] * inv;
                x[3] = oacc[db][4 * g + 3] * inv;
                *reinterpret_cast<floatx4*>(orow + d) = x;
            }
        if (h == 0) LSE[(int64_t)bh * M + query] = (m_run + fast_log2(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// host side: validation, dispatch table, launch
// ---------------------------------------------------------------------------
struct LaunchArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int BH, M, N;
    float c_log2;
};

typedef hipError_t (*launch_fn)(const LaunchArgs&, hipStream_t);

template <int D, int BN, int NW, int QB, bool CAUSAL>
hipError_t launch_bf16(const LaunchArgs& a, hipStream_t stream) {
    using T = Bf16Traits<D, BN, NW, QB>;
    const int n_qt = (a.M + T::kBM - 1) / T::kBM;
    const __bf16* q = static_cast<const __bf16*>(a.q);
    const __bf16* k = static_cast<const __bf16*>(a.k);
    const __bf16* v = static_cast<const __bf16*>(a.v);
    __bf16* o = static_cast<__bf16*>(a.o);
    float* lse = a.lse;
    int BH = a.BH, M = a.M, N = a.N;
    float c = a.c_log2;
    void* args[] = {&q, &k, &v, &o, &lse, &BH, &M, &N, (void*)&n_qt, &c};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fa2_fwd_bf16_kernel<D, BN, NW, QB, CAUSAL>),
                           dim3((unsigned)(n_qt * a.BH)), dim3(T::kThreads), args, 0, stream);
}

template <int D, int BN, int NW, bool CAUSAL>
hipError_t launch_f32(const LaunchArgs& a, hipStream_t stream) {
    using T = F32Traits<D, BN, NW>;
    const int n_qt = (a.M + T::kBM - 1) / T::kBM;
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    float* o = static_cast<float*>(a.o);
    float* lse = a.lse;
    int BH = a.BH, M = a.M, N = a.N;
    float c = a.c_log2;
    void* args[] = {&q, &k, &v, &o, &lse, &BH, &M, &N, (void*)&n_qt, &c};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fa2_fwd_f32_kernel<D, BN, NW, CAUSAL>),
                           dim3((unsigned)(n_qt * a.BH)), dim3(T::kThreads), args, 0, stream);
}

// Dispatch on (dtype, head dim, causal), as the pages' C++ entry point does
// with its dtype/head-dim/bool switches; each entry is one compiled kernel.
struct Entry {
    int dtype, D, causal;
    launch_fn fn;
    int block_m;
};

const Entry kTable[] = {
    {FA2_DTYPE_BF16, 64, 0, &launch_bf16<64, 64, 4, 1, false>, 128},
    {FA2_DTYPE_BF16, 64, 1, &launch_bf16<64, 64, 4, 1, true>, 128},
    {FA2_DTYPE_BF16, 128, 0, &launch_bf16<128, 64, 4, 1, false>, 128},
    {FA2_DTYPE_BF16, 128, 1, &launch_bf16<128, 64, 4, 1, true>, 128},
    {FA2_DTYPE_F32, 64, 0, &launch_f32<64, 64, 4, false>, 128},
    {FA2_DTYPE_F32, 64, 1, &launch_f32<64, 64, 4, true>, 128},
    {FA2_DTYPE_F32, 128, 0, &launch_f32<128, 32, 4, false>, 128},
    {FA2_DTYPE_F32, 128, 1, &launch_f32<128, 32, 4, true>, 128},
};

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                       float scale, int causal, int dtype, void* stream) {
    // ---- argument checks, all before any HIP call
    if (!q || !k || !v || !o || !lse) return FA2_ERR_INVALID_ARGUMENT;
    if (B < 0 || H < 0 || M < 0 || N <= 0 || D <= 0) return FA2_ERR_INVALID_ARGUMENT;
    if (dtype != FA2_DTYPE_F32 && dtype != FA2_DTYPE_BF16) return FA2_ERR_INVALID_ARGUMENT;
    if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARGUMENT;
    if (!(scale > 0.f) || !isfinite(scale)) return FA2_ERR_INVALID_ARGUMENT;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(lse, 4))
        return FA2_ERR_INVALID_ARGUMENT;

    const Entry* e = nullptr;
    for (const Entry& t : kTable)
        if (t.dtype == dtype && t.D == D && t.causal == causal) e = &t;
    if (!e) return FA2_ERR_UNSUPPORTED;

    // sizes: per-head offsets are 32-bit in the kernels, the grid is 1-D
    const int64_t kMax = (int64_t)1 << 31;
    if (B > kMax || H > kMax) return FA2_ERR_UNSUPPORTED;
    const int64_t BH = B * H;
    if (M * D >= kMax || N * D >= kMax || BH >= kMax) return FA2_ERR_UNSUPPORTED;
    const int64_t n_qt = (M + e->block_m - 1) / e->block_m;
    if (n_qt * BH >= kMax) return FA2_ERR_UNSUPPORTED;

    const size_t elt = dtype == FA2_DTYPE_F32 ? 4 : 2;
    const size_t o_bytes = (size_t)BH * M * D * elt;
    const size_t kv_bytes = (size_t)BH * N * D * elt;
    const size_t lse_bytes = (size_t)BH * M * 4;
    if (overlaps(o, o_bytes, q, o_bytes) || overlaps(o, o_bytes, k, kv_bytes) ||
        overlaps(o, o_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, q, o_bytes) ||
        overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes) ||
        overlaps(lse, lse_bytes, o, o_bytes))
        return FA2_ERR_INVALID_ARGUMENT;

    if (M == 0 || BH == 0) return FA2_OK;

    LaunchArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.BH = (int)BH; a.M = (int)M; a.N = (int)N;
    a.c_log2 = scale * 1.44269504088896340736f;  // scale * log2(e)
    const hipError_t err = e->fn(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

extern "C" const char* fa2_status_string(int status) {
    switch (status) {
        case FA2_OK: return "FA2_OK: success";
        case FA2_ERR_INVALID_ARGUMENT: return "FA2_ERR_INVALID_ARGUMENT: null, misaligned or overlapping pointer, or bad size, dtype, causal flag or scale";
        case FA2_ERR_UNSUPPORTED: return "FA2_ERR_UNSUPPORTED: head dimension or problem size not supported by this build";
        case FA2_ERR_LAUNCH: return "FA2_ERR_LAUNCH: the HIP runtime rejected the kernel launch";
        case FA2_ERR_NO_DEVICE: return "FA2_ERR_NO_DEVICE: no usable gfx950 device";
        default: return "unknown fa2 status";
    }
}
