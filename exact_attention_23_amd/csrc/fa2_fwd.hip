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
//    unnormalised O, all fp32, rescaled by exp(m_old - m_new) when the max
//    moves ("FlashAttention-2 from PyTorch to Triton", the tile loop and the
//    accumulator discussion; "Writing FlashAttention 2 in Triton", Step 4);
//    the kernels move it only when the weights would otherwise leave the
//    range their formats hold (see the kernels), which changes rounding only;
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
//    MFMA (lane = query, 8 keys per lane).  The A operand, V^T, is read from a
//    row-major LDS copy of V with ds_read_b64_tr_b16 (bf16), or one key per
//    lane with plain reads (fp32).
//  * K and V tiles are copied global -> LDS by the load unit (buffer loads
//    with the LDS bit, 16 bytes per lane, no VGPR staging) into unpadded
//    rows with XOR-swizzled 16-byte chunks, double-buffered; the next tile's
//    copies are issued before the current tile's MFMAs.
//  * Q stays in VGPRs for the whole K/V loop; O^T, m, l stay in registers.
//  * Causal grids launch the heaviest query tiles first; batch*head is the
//    fastest-varying grid index so that all tiles of one head land on the same
//    XCD (workgroups are dealt to the 8 XCDs round-robin).
//  * the dense 16-bit path uses a ping-pong schedule between two groups of
//    four waves (see fa2_fwd_half_pp_kernel): one wave of a SIMD runs MFMAs
//    while the other runs the softmax.

#include <hip/hip_runtime.h>
#include <math.h>
#include <type_traits>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "fa2.h"
#include "fa2_common.h"

namespace {

// ---------------------------------------------------------------------------
// parameters and work assignment shared by the forward kernels
// ---------------------------------------------------------------------------
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    float* ws_o;          // split K/V: partial O [n_splits, BH, M, D] fp32, else null
    float* ws_l;          // split K/V: partial L [n_splits, BH, M] fp32, else null
    const int* cu_q;      // packed sequences: query row offsets [B + 1] (device), else null
    const int* cu_k;      // packed sequences: key row offsets [B + 1]
    int total_q, total_k; // packed sequences: rows per head of q (o, lse) and of k (v)
    int BH;               // batch * query heads
    int H;                // query heads
    int Hk;               // K/V heads
    int G;                // query heads per K/V head (H / Hk)
    int M, N;             // dense: query rows and keys per head
    int n_qt;             // query tiles per head
    int tiles_per_split;  // K/V tiles per split (at least all of them when unsplit)
    int wl, wr;           // sliding window: keys i - wl .. i + wr (-1: unbounded side)
    float c_log2;         // scale * log2(e)
};

// First and last key query row i of a sequence of N keys sees (lo > hi: none).
template <int MASK>
__device__ __forceinline__ int key_lo(const FwdParams& p, int i) {
    return key_lo<MASK>(p.wl, i);
}
template <int MASK>
__device__ __forceinline__ int key_hi(const FwdParams& p, int i, int N) {
    return key_hi<MASK>(p.wr, i, N);
}

// The (batch, head) sequence a workgroup works on: a head of the dense
// [B, H, M, D] layout (cu_q == null), or sequence b of the packed layout
// [H, total_q, D] / [Hk, total_k, D] whose rows cu_q[b] .. cu_q[b + 1] - 1
// (keys cu_k[b] .. cu_k[b + 1] - 1) belong to it.  Offsets outside
// [0, total] are clamped, so a malformed offset array cannot address memory
// past the tensors.
struct SeqView {
    int64_t q_row0;   // row of q, o and lse that holds the sequence's query 0
    int64_t kv_row0;  // row of k and v that holds its key 0
    int M, N;         // query rows and keys of the sequence
};
__device__ __forceinline__ SeqView seq_view(const FwdParams& p, int bh, int bkv) {
    SeqView v;
    if (p.cu_q == nullptr) {
        v.M = p.M;
        v.N = p.N;
        v.q_row0 = (int64_t)bh * p.M;
        v.kv_row0 = (int64_t)bkv * p.N;
    } else {
        const int b = bh / p.H, h = bh - b * p.H, hk = bkv - b * p.Hk;
        const int q0 = min(max(p.cu_q[b], 0), p.total_q), q1 = min(max(p.cu_q[b + 1], q0), p.total_q);
        const int k0 = min(max(p.cu_k[b], 0), p.total_k), k1 = min(max(p.cu_k[b + 1], k0), p.total_k);
        v.M = q1 - q0;
        v.N = k1 - k0;
        v.q_row0 = (int64_t)h * p.total_q + q0;
        v.kv_row0 = (int64_t)hk * p.total_k + k0;
    }
    return v;
}

// One workgroup's task: query tile qt of sequence sv (head bh), reading K/V
// head bkv (query head h uses K/V head h / G, "From FlashAttention to
// FlashAttention 2", section "Layer 8"), over K/V tiles
// [t_begin, t_begin + n_kv) of its split.
struct WgTask {
    int bh, bkv, qt, split;
    SeqView sv;
    int t_begin;  // first K/V tile of the workgroup (of its split)
    int n_kv;     // K/V tiles of this workgroup (0 for a split past the diagonal)
};

// Grid order: split-major, then query tile (heaviest first when causal), then
// batch*head fastest, so that the tiles of one head spread over the XCDs in
// step and every XCD gets the same mix of heavy and light tiles.  The tiles a
// workgroup needs run from the first key its first row sees to the last key
// its last row sees.
template <int MASK, bool SPLIT>
__device__ __forceinline__ WgTask wg_task(const FwdParams& p, int BM, int BN) {
    WgTask t;
    const int wg = blockIdx.x;
    int r = wg;
    t.split = 0;
    if (SPLIT) {
        const int per_split = p.BH * p.n_qt;
        t.split = wg / per_split;
        r = wg - t.split * per_split;
    }
    t.bh = r % p.BH;
    t.qt = r / p.BH;
    if (MASK == kMaskCausal) t.qt = p.n_qt - 1 - t.qt;
    // bh = (b * Hk + hk) * G + g for query head h = hk * G + g
    t.bkv = p.G == 1 ? t.bh : t.bh / p.G;
    t.sv = seq_view(p, t.bh, t.bkv);
    const int r0 = t.qt * BM, r1 = min(r0 + BM, t.sv.M) - 1;
    int lo_t = 0, hi_t = 0;  // the query tile's K/V tiles [lo_t, hi_t)
    if (r0 <= r1) {
        const int klo = key_lo<MASK>(p, r0), khi = key_hi<MASK>(p, r1, t.sv.N);
        if (klo <= khi) {
            lo_t = klo / BN;
            hi_t = khi / BN + 1;
        }
    }
    t.t_begin = lo_t + t.split * p.tiles_per_split;
    t.n_kv = max(0, min(hi_t - t.t_begin, p.tiles_per_split));
    return t;
}

// The workgroup's K/V tiles [first, end) (indices from t_begin) that a wave
// whose rows start at qw0 needs: each row only needs the tiles of its keys;
// rows past M need none.
struct WaveRange {
    int first, end;
};
template <int MASK>
__device__ __forceinline__ WaveRange wave_tiles(const FwdParams& p, const WgTask& t, int qw0, int rows, int BN) {
    WaveRange w{0, 0};
    const int r1 = min(qw0 + rows, t.sv.M) - 1;
    if (qw0 > r1) return w;
    const int klo = key_lo<MASK>(p, qw0), khi = key_hi<MASK>(p, r1, t.sv.N);
    if (klo > khi) return w;
    w.first = max(klo / BN - t.t_begin, 0);
    w.end = max(min(khi / BN + 1 - t.t_begin, t.n_kv), w.first);
    return w;
}

// Does K/V tile kbase .. kbase + BN - 1 need a mask for the rows qa .. qb of a
// wave: it runs past N, or past the last key of the first row, or starts
// before the first key of the last row.
template <int MASK>
__device__ __forceinline__ bool tile_needs_mask(const FwdParams& p, int kbase, int BN, int N, int qa, int qb) {
    if (kbase + BN > N) return true;
    if (MASK != kMaskNone && kbase + BN - 1 > key_hi<MASK>(p, qa, N)) return true;
    if (MASK == kMaskLocal && kbase < key_lo<MASK>(p, qb)) return true;
    return false;
}

// Split-K/V partial result of one query row (the lane's 4 consecutive O values
// at d): O normalised by the split's own sum, and the split's L (-inf when the
// split saw no visible key; its O is then 0).
__device__ __forceinline__ float* partial_row(const FwdParams& p, const WgTask& t, int query, int D) {
    return p.ws_o + (((int64_t)t.split * p.BH + t.bh) * p.M + query) * D;
}
__device__ __forceinline__ float* partial_l(const FwdParams& p, const WgTask& t, int query) {
    return p.ws_l + ((int64_t)t.split * p.BH + t.bh) * p.M + query;
}

// ---------------------------------------------------------------------------
// 16-bit kernel (bf16 or fp16 inputs, E)
// ---------------------------------------------------------------------------
// D: head dim (64 or 128); BN: keys per K/V tile (multiple of 32);
// NW: waves per workgroup; QB: 32-query blocks per wave.
//
// K and V tiles are copied global -> LDS by the load unit itself
// (buffer_load_dwordx4 ... lds: each lane moves one 16-byte chunk, a wave
// fills 1 KiB of LDS), so no VGPRs stage them.  Rows are stored unpadded with their
// 16-byte chunks XOR-permuted per row (the lane -> global address map does the
// permutation), which keeps both read patterns free of bank conflicts:
//  * K is read as the A operand of S^T = K Q^T: lanes 0..31 read 32 different
//    key rows at one logical chunk -> chunk ^= f_K(row) spreads them;
//  * V is read with ds_read_b64_tr_b16, which hands each lane 4 consecutive
//    keys of one d column (a 4-key x 16-d block per 16 lanes transposed in
//    flight) -- exactly the A operand of O^T += V^T P^T -- so V needs no
//    transposition in LDS; chunk ^= f_V(row) keeps the 4 rows x 64 bytes a
//    half-wave reads in distinct banks.
template <int D, int BN, int NW, int QB>
struct HalfTraits {
    static constexpr int kThreads = NW * 64;
    static constexpr int kQPW = 32 * QB;          // query rows per wave
    static constexpr int kBM = kQPW * NW;         // query rows per workgroup
    static constexpr int kKB = BN / 32;           // 32-key blocks per tile
    static constexpr int kDB = D / 32;            // 32-wide d blocks of O^T
    static constexpr int kDS = D / 16;            // MFMA k-steps of S^T
    static constexpr int kCPR = D / 8;            // 16-byte chunks per row
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = BN * kRowBytes;
    static constexpr int kTileChunks = BN * kCPR;
    static constexpr int kLoadsPerWave = kTileChunks / (64 * NW);  // per tensor per tile
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BN % 32 == 0, "key tile");
    static_assert(kTileChunks % (64 * NW) == 0, "loader split");
};

// s_waitcnt operand that waits until at most n (0 <= n < 64) vector-memory
// operations of this wave are outstanding and leaves the other counters alone
// (vmcnt in bits 3:0 and 15:14, expcnt 7, lgkmcnt 15).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xf00; }

// XOR applied to the 16-byte chunk index of LDS row r (K tile): the 16 rows a
// quarter-wave reads at one logical chunk land in 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
// XOR for the V tile: rows key0..key0+3 (key0 % 4 == 0) read 64 bytes each at
// one set of 4 logical chunks; the XOR moves each row's 64 bytes to its own
// quarter of the 256-byte bank space.
template <int D>
__device__ __forceinline__ int swz_v(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}


// BUFS: K/V tile buffer pairs, 2 (double buffering) or 4 (a ring with three
// tiles' copies in flight, for long key ranges).
template <typename E, int D, int BN, int NW, int QB, int WAVES_PER_SIMD, int BUFS, int MASK, bool SPLIT>
__global__ void __launch_bounds__(NW * 64, WAVES_PER_SIMD)
fa2_fwd_half_kernel(const FwdParams p) {
    static_assert(BUFS == 2 || BUFS == 4, "buffer pairs");
    using T = HalfTraits<D, BN, NW, QB>;
    using V8 = typename Half<E>::v8;
    using V2 = typename Half<E>::v2;
    const E* __restrict__ Q = static_cast<const E*>(p.q);
    const E* __restrict__ K = static_cast<const E*>(p.k);
    const E* __restrict__ V = static_cast<const E*>(p.v);
    E* __restrict__ O = static_cast<E*>(p.o);
    float* __restrict__ LSE = p.lse;
    const float c_log2 = p.c_log2;
    // K/V tile buffers, each BN rows x D (rows unpadded, chunks swizzled).
    // They are separate arrays, and the loops below are unrolled over them so
    // every access names its buffer statically: the compiler can then see
    // that the asynchronous copies into the other buffers never alias the
    // reads of one, and does not stall those reads on the copies.  (The ring
    // form declares its third and fourth pairs with its loop.)
    __shared__ __attribute__((aligned(1024))) char sK0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sK1[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV1[T::kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    const WgTask task = wg_task<MASK, SPLIT>(p, T::kBM, BN);
    const int M = task.sv.M, N = task.sv.N;
    const int qw0 = task.qt * T::kBM + wave * T::kQPW;  // first query row of this wave
    const int qw1 = min(qw0 + T::kQPW, M) - 1;          // last one

    const E* Qh = Q + task.sv.q_row0 * D;
    const E* Kh = K + task.sv.kv_row0 * D;
    const E* Vh = V + task.sv.kv_row0 * D;

    // local tile kt is K/V tile kv_t0 + kt of the head
    const int kv_t0 = task.t_begin;
    const int n_kv = task.n_kv;
    const WaveRange wtiles = wave_tiles<MASK>(p, task, qw0, T::kQPW, BN);

    // ---- Q fragments: B operand of S^T = K Q^T (lane = query, 8 d values)
    V8 qf[QB][T::kDS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw0 + 32 * qb + l32;
#pragma unroll
        for (int s = 0; s < T::kDS; ++s) {
            if (row < M) {
                qf[qb][s] = *reinterpret_cast<const V8*>(Qh + (int64_t)row * D + 16 * s + 8 * h);
            } else {
                qf[qb][s] = V8{};
            }
        }
    }

    // Running state per query row (one row per lane): O^T accumulators, the
    // max m (log2 units), and two partial sums of this lane's weights: l_run
    // over the bf16-rounded weights the PV MFMA consumed (the denominator of
    // O), l_exact over the fp32 weights (for L = m + log l).
    floatx16 oacc[T::kDB][QB];
    float m_run[QB], l_run[QB], l_exact[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
        l_exact[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db) oacc[db][qb] = floatx16{};
    }

    // ---- async tile copy: wave w moves chunks [w*L*64, (w+1)*L*64) of each
    // tensor's tile; LDS slot s holds row s / CPR, physical chunk s % CPR,
    // i.e. logical chunk (s % CPR) ^ swz(row).
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t cp_koff[T::kLoadsPerWave], cp_voff[T::kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < T::kLoadsPerWave; ++i) {
        const int slot = (wave * T::kLoadsPerWave + i) * 64 + lane;
        const int r = slot / T::kCPR, p = slot % T::kCPR;
        cp_koff[i] = (uint32_t)(r * T::kRowBytes + 16 * (p ^ swz_k<D>(r)));
        cp_voff[i] = (uint32_t)(r * T::kRowBytes + 16 * (p ^ swz_v<D>(r)));
    }
    auto issue_tile = [&](int kt, char* kdst, char* vdst) {
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BN>(Kh, cp_koff, wave_u, kv_t0 + kt, N, kdst);
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BN>(Vh, cp_voff, wave_u, kv_t0 + kt, N, vdst);
    };

    // per-lane parts of the LDS fragment addresses
    // K (A operand of S^T): row 32 kb + l32, logical chunk 2 s + h.
    int k_lane_off[T::kDS];
#pragma unroll
    for (int s = 0; s < T::kDS; ++s)
        k_lane_off[s] = l32 * T::kRowBytes + 16 * ((2 * s + h) ^ swz_k<D>(l32));
    // V^T (A operand of O^T += V^T P^T) via ds_read_b64_tr_b16: lane
    // 16 g + 4 t + a reads row key0 + t, d = d0 + 4a, where the 16-lane group g
    // covers d0 = 32 db + 16 (g & 1) and key0 = ... + 4 (g >> 1).
    const int vg = lane >> 4, vt = (lane >> 2) & 3, va = lane & 3;
    const int v_row_lane = 4 * (vg >> 1) + vt;
    int v_lane_off[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) {
        const int c = 4 * db + 2 * (vg & 1) + (va >> 1);
        v_lane_off[db] = v_row_lane * T::kRowBytes + 16 * (c ^ swz_v<D>(v_row_lane)) + 8 * (va & 1);
    }

    // kt: K/V tile of the head (only the mask uses it)
    auto compute_tile = [&](auto mask_tag, int kt, const char* klds, const char* vlds) {
        constexpr bool BOUNDARY = decltype(mask_tag)::value;
        // S^T = K Q^T for BN keys x QPW queries; K fragments are read one
        // k-step ahead of the MFMAs that use them.
        floatx16 sacc[T::kKB][QB];
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = floatx16{};
        V8 kf[2][T::kKB];
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
            kf[0][kb] = *reinterpret_cast<const V8*>(klds + 32 * kb * T::kRowBytes + k_lane_off[0]);
#pragma unroll
        for (int s = 0; s < T::kDS; ++s) {
            if (s + 1 < T::kDS) {
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
                    kf[(s + 1) & 1][kb] = *reinterpret_cast<const V8*>(
                        klds + 32 * kb * T::kRowBytes + k_lane_off[s + 1]);
            }
            // keep the next step's reads ahead of this step's MFMAs
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    sacc[kb][qb] = Half<E>::mfma(kf[s & 1][kb], qf[qb][s], sacc[kb][qb]);
        }

        // boundary tiles only: keys past N, and keys outside the query's
        // causal or window range.  Key kbase + 32 kb + acc_row(r, h) is
        // visible iff its compile-time part 32 kb + 8 (r / 4) + r % 4 lies in
        // [lim_lo, lim].
        if constexpr (BOUNDARY) {
            const int kbase = kt * BN;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int query = qw0 + 32 * qb + l32;
                const int lim = key_hi<MASK>(p, query, N) - kbase - 4 * h;
                const int lim_lo = key_lo<MASK>(p, query) - kbase - 4 * h;
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int idx = 32 * kb + 8 * (r >> 2) + (r & 3);
                        if (idx > lim || (MASK == kMaskLocal && idx < lim_lo)) sacc[kb][qb][r] = -INFINITY;
                    }
            }
        }

        V8 pf[T::kKB][2][QB];  // P^T as B operands of the PV MFMAs
        // Online softmax in the log2 domain.  The weights are first taken
        // against the running max as it stands, P = exp2(s*c - m_run); the
        // max only has to move when some weight would leave the range of the
        // 16-bit P (and of fp32 O and l), which the lane's sum of P shows
        // after the fact: a sum above Half<E>::kWeightSumCap, an inf, or the
        // NaN of a row with no max yet fails the test, and only then is the
        // tile's row max taken, O and l rescaled and P recomputed.  Large
        // weights lose nothing (fp32 O and l and the 16-bit P are relative
        // formats; the key that last set the max had weight 1, so l >= 1).
        // P is rounded once, for the PV MFMA.  l_run sums exactly those
        // rounded weights (two per v_dot2 against (1, 1)), so O / l_run is a
        // true weighted mean of V rows; l_exact sums the fp32 weights, which
        // L needs to within 1e-3.
        auto weights = [&](int qb, float m_sub, float& lr, float& le) {
            float lsum = 0.f, esum = 0.f;
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                    for (int t = 0; t < 8; t += 2) {
                        const float p0 = fast_exp2(fmaf(sacc[kb][qb][8 * ms + t], c_log2, -m_sub));
                        const float p1 = fast_exp2(fmaf(sacc[kb][qb][8 * ms + t + 1], c_log2, -m_sub));
                        const V2 pp = {(E)p0, (E)p1};
                        pf[kb][ms][qb][t] = pp[0];
                        pf[kb][ms][qb][t + 1] = pp[1];
                        lsum = Half<E>::sum2(pp, lsum);
                        esum += p0;
                        esum += p1;
                    }
            lr = lsum;
            le = esum;
        };
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float lr, le;
            weights(qb, m_run[qb], lr, le);
            if (__any(!(le <= Half<E>::kWeightSumCap))) {  // (not ">": NaN must fail too)
                // (the empty volatile asm keeps the compiler from turning this
                // rarely taken branch into always-executed selects)
                __asm__ volatile("");
                // IEEE maximum (v_maximum3_f32): no NaN quieting of each input
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; r += 2)
                        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(sacc[kb][qb][r], sacc[kb][qb][r + 1]));
                {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                    mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                }
                const float m_new = fmaxf(m_run[qb], mx * c_log2);
                const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run[qb] - m_new);
                m_run[qb] = m_new;
                l_run[qb] *= alpha;
                l_exact[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) oacc[db][qb] *= alpha;
                weights(qb, m_new == -INFINITY ? 0.f : m_new, lr, le);
            }
            l_run[qb] += lr;
            l_exact[qb] += le;
        }

        // O^T += V^T P^T: two 16-key MFMA steps per 32-key block; each A
        // operand is two transposed 4-key reads, issued one step ahead.
        constexpr int kSteps = T::kKB * 2;
        auto read_v = [&](int step, int db) {
            const char* p0 = vlds + 16 * step * T::kRowBytes + v_lane_off[db];
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 8 * T::kRowBytes));
            return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        V8 vf[2][T::kDB];
#pragma unroll
        for (int db = 0; db < T::kDB; ++db) vf[0][db] = read_v(0, db);
#pragma unroll
        for (int step = 0; step < kSteps; ++step) {
            if (step + 1 < kSteps) {
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) vf[(step + 1) & 1][db] = read_v(step + 1, db);
            }
            const int kb = step >> 1, ms = step & 1;
#pragma unroll
            for (int db = 0; db < T::kDB; ++db)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    oacc[db][qb] = Half<E>::mfma(vf[step & 1][db], pf[kb][ms][qb], oacc[db][qb]);
        }
    };

    // A tile needs masking if it runs past N or cuts into some row's causal
    // or window range; all other tiles take the mask-free path.
    auto run_tile = [&](int kt, const char* klds, const char* vlds) {
        if (kt < wtiles.first || kt >= wtiles.end) return;
        const int kbase = (kv_t0 + kt) * BN;
        if (tile_needs_mask<MASK>(p, kbase, BN, N, qw0, qw1))
            compute_tile(std::true_type{}, kv_t0 + kt, klds, vlds);
        else
            compute_tile(std::false_type{}, kv_t0 + kt, klds, vlds);
    };
    if constexpr (BUFS == 2) {
        // ---- main loop, unrolled by two over the buffer pair
        if (n_kv > 0) issue_tile(0, sK0, sV0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int kt = 0; kt < n_kv; kt += 2) {
            if (kt + 1 < n_kv) issue_tile(kt + 1, sK1, sV1);
            run_tile(kt, sK0, sV0);
            __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next tile have landed
            __syncthreads();
            if (kt + 1 >= n_kv) break;
            if (kt + 2 < n_kv) issue_tile(kt + 2, sK0, sV0);
            run_tile(kt + 1, sK1, sV1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    } else {
        // ---- main loop over a ring of four buffer pairs, unrolled by four:
        // tile kt + 3 is issued into the buffer tile kt - 1 left before tile
        // kt is computed, so three tiles' copies are in flight.  Before the
        // barrier that hands tile kt + 1 to the waves, a wave waits for its
        // own copies of that tile only: a wave's buffer loads count its
        // vector-memory counter down in issue order, so at most
        // j * kLoadsPerTile outstanding means all but the j newest tiles have
        // landed (any other load of the wave only lengthens the wait).  The
        // barrier also tells the wave that issues next into a buffer that the
        // other waves have finished reading it.
        __shared__ __attribute__((aligned(1024))) char sK2[T::kTileBytes];
        __shared__ __attribute__((aligned(1024))) char sV2[T::kTileBytes];
        __shared__ __attribute__((aligned(1024))) char sK3[T::kTileBytes];
        __shared__ __attribute__((aligned(1024))) char sV3[T::kTileBytes];
        constexpr int kLoadsPerTile = 2 * T::kLoadsPerWave;  // a wave's copies of one K and one V tile
        auto wait_for_next = [&](int kt) {  // after tile kt: tile kt + 1 has landed
            const int newer = min(n_kv - 1, kt + 3) - (kt + 1);  // tiles issued after kt + 1
            if (newer >= 2)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kLoadsPerTile));
            else if (newer == 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_only(kLoadsPerTile));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            lds_barrier();
        };
        if (n_kv > 0) issue_tile(0, sK0, sV0);
        if (n_kv > 1) issue_tile(1, sK1, sV1);
        if (n_kv > 2) issue_tile(2, sK2, sV2);
        wait_for_next(-1);
        for (int kt = 0; kt < n_kv; kt += 4) {
            if (kt + 3 < n_kv) issue_tile(kt + 3, sK3, sV3);
            run_tile(kt, sK0, sV0);
            if (kt + 1 >= n_kv) break;
            wait_for_next(kt);
            if (kt + 4 < n_kv) issue_tile(kt + 4, sK0, sV0);
            run_tile(kt + 1, sK1, sV1);
            if (kt + 2 >= n_kv) break;
            wait_for_next(kt + 1);
            if (kt + 5 < n_kv) issue_tile(kt + 5, sK1, sV1);
            run_tile(kt + 2, sK2, sV2);
            if (kt + 3 >= n_kv) break;
            wait_for_next(kt + 2);
            if (kt + 6 < n_kv) issue_tile(kt + 6, sK2, sV2);
            run_tile(kt + 3, sK3, sV3);
            if (kt + 4 >= n_kv) break;
            wait_for_next(kt + 3);
        }
    }

    // ---- epilogue: one normalisation, L = (m + log2 l) * ln 2, RNE store
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[qb]), __float_as_uint(l_run[qb]), false, false);
        const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const auto se = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_exact[qb]), __float_as_uint(l_exact[qb]), false, false);
        const float l_ex = __uint_as_float(se[0]) + __uint_as_float(se[1]);
        const int query = qw0 + 32 * qb + l32;
        if (query < M) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            const float lse = (m_run[qb] + fast_log2(l_ex)) * kLn2;
            if constexpr (SPLIT) {
                float* orow = partial_row(p, task, query, D);
#pragma unroll
                for (int db = 0; db < T::kDB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const floatx4 x = {oacc[db][qb][4 * g + 0] * inv, oacc[db][qb][4 * g + 1] * inv,
                                           oacc[db][qb][4 * g + 2] * inv, oacc[db][qb][4 * g + 3] * inv};
                        *reinterpret_cast<floatx4*>(orow + 32 * db + 8 * g + 4 * h) = x;
                    }
                if (h == 0) *partial_l(p, task, query) = lse;
            } else {
                E* orow = O + (task.sv.q_row0 + query) * D;
#pragma unroll
                for (int db = 0; db < T::kDB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int d = 32 * db + 8 * g + 4 * h;
                        uint32_t w[2];
                        w[0] = pack2<E>(oacc[db][qb][4 * g + 0] * inv, oacc[db][qb][4 * g + 1] * inv);
                        w[1] = pack2<E>(oacc[db][qb][4 * g + 2] * inv, oacc[db][qb][4 * g + 3] * inv);
                        *reinterpret_cast<uint2*>(orow + d) = make_uint2(w[0], w[1]);
                    }
                if (h == 0) LSE[task.sv.q_row0 + query] = lse;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 16-bit kernel, ping-pong schedule
// ---------------------------------------------------------------------------
// A wave issues in order, so its softmax overlaps its own MFMAs only when
// the two are interleaved instruction by instruction; the MFMA of one wave
// and the VALU of another wave on the same SIMD overlap without that.  This
// kernel runs two groups of four waves (waves w and w + 4 share a SIMD) half
// a tile out of phase:
//
//   period:     0        1        2          3          4 ...
//   group A:  S(0)     sm(0)    PV(0)+S(1)  sm(1)      PV(1)+S(2)
//   group B:  -        S(0)     sm(0)      PV(0)+S(1)  sm(1)
//
// where S(t) = K_t Q^T and PV(t) = O^T += V_t^T P_t^T are MFMA-only phases and
// sm(t) (mask, online softmax, rescale) is VALU-only, so while one wave of a
// SIMD keeps the matrix core busy the other wave uses the vector ALU.
//
// K_t is read in periods 2t (A) and 2t+1 (B), V_t in 2t+2 (A) and 2t+3 (B).
// At the start of each even period 2t every wave issues its share of the
// copies of K_{t+1} and V_t; it waits for them before the workgroup barrier
// that ends period 2t+1, one period before they are read.  That barrier, one
// per tile, is the only one: it publishes those copies and retires the reads
// of K_t and V_{t-1}, whose buffers the next copies overwrite; between two
// barriers group A runs its MFMA phase then its softmax, group B its softmax
// then its MFMA phase, with nothing to keep them in step (a barrier there
// would guard no buffer).  K_t and V_t live in buffer t % 2; the loop is
// unrolled over four periods so that every LDS access names its buffer
// statically and the compiler can see that the copies in flight never alias
// the buffers being read.  The four buffers (64 KiB at D = 128) fill the
// bottom of LDS, so each buffer's base fits a DS instruction's 16-bit
// immediate offset and an operand read is a single instruction; a buffer
// above 64 KiB would cost an address add per read, in the MFMA phase.
//
// Each wave owns 32 query rows; group A takes the even 32-row blocks of the
// workgroup's 256 rows and group B the odd ones, so under a causal mask the
// two waves of a SIMD need the same number of tiles (to within one).  The
// kernel serves the dense, sliding-window and packed-sequence calls: under a
// window a wave's rows see keys from tile w_first on, and the tiles before
// it give P = 0 without a softmax.
template <int D, int BN>
struct PPTraits {
    static constexpr int kNW = 8;
    static constexpr int kThreads = kNW * 64;
    static constexpr int kBM = 32 * kNW;          // query rows per workgroup
    static constexpr int kKB = BN / 32;           // 32-key blocks per tile
    static constexpr int kDB = D / 32;            // 32-wide d blocks of O^T
    static constexpr int kDS = D / 16;            // MFMA k-steps of S^T
    static constexpr int kCPR = D / 8;            // 16-byte chunks per row
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = BN * kRowBytes;
    static constexpr int kTileChunks = BN * kCPR;
    static constexpr int kLoadsPerWave = kTileChunks / (64 * kNW);  // per tensor per tile
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BN % 32 == 0, "key tile");
    static_assert(kTileChunks % (64 * kNW) == 0, "loader split");
};

template <typename E, int D, int BN, int MASK, bool SPLIT, bool PACKED = false>
__global__ void __launch_bounds__(512, 2)
fa2_fwd_half_pp_kernel(const FwdParams p) {
    using T = PPTraits<D, BN>;
    using V8 = typename Half<E>::v8;
    using V2 = typename Half<E>::v2;
    const E* __restrict__ Q = static_cast<const E*>(p.q);
    const E* __restrict__ K = static_cast<const E*>(p.k);
    const E* __restrict__ V = static_cast<const E*>(p.v);
    E* __restrict__ O = static_cast<E*>(p.o);
    float* __restrict__ LSE = p.lse;
    const float c_log2 = p.c_log2;
    __shared__ __attribute__((aligned(1024))) char sK0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sK1[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV1[T::kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = wave >> 2;  // 0: group A, 1: group B
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // the workgroup's sequence: a head of the dense layout or one packed
    // sequence; any mask kind (none, causal, sliding window)
    const WgTask task = wg_task<MASK, SPLIT>(p, T::kBM, BN);
    const int M = task.sv.M, N = task.sv.N;
    // packed sequences: a query tile past its sequence's rows (sequences
    // shorter than the longest) has nothing to compute or store; the
    // condition is the same for every wave of the workgroup, so no barrier
    // is left waiting.  (Compiled only into the packed form: in the others
    // the test cost ~1 % on the dense shapes.)
    if constexpr (PACKED) {
        if (task.qt * T::kBM >= M) return;
    }
    const int qw0 = task.qt * T::kBM + 32 * (2 * (wave & 3) + grp);  // first query row of this wave
    const int qw1 = min(qw0 + 32, M) - 1;                             // its last one

    const E* Qh = Q + task.sv.q_row0 * D;
    const E* Kh = K + task.sv.kv_row0 * D;
    const E* Vh = V + task.sv.kv_row0 * D;

    // local tile t is K/V tile kv_t0 + t of the head; the wave's rows see
    // keys in tiles [w_first, n_w) only (w_first > 0 under a window)
    const int kv_t0 = task.t_begin;
    const int n_kv = task.n_kv;
    const WaveRange w_range = wave_tiles<MASK>(p, task, qw0, 32, BN);
    const int n_w = w_range.end, w_first = w_range.first;

    // ---- Q fragments: B operand of S^T = K Q^T (lane = query, 8 d values)
    V8 qf[T::kDS];
    {
        const int row = qw0 + l32;
#pragma unroll
        for (int s = 0; s < T::kDS; ++s)
            qf[s] = row < M ? *reinterpret_cast<const V8*>(Qh + (int64_t)row * D + 16 * s + 8 * h)
                            : V8{};
    }

    // Running state of this lane's query row: O^T, the max m (log2 units),
    // l_run over the bf16-rounded weights the PV MFMA consumed (denominator of
    // O) and l_exact over the fp32 weights (for L).
    floatx16 oacc[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) oacc[db] = floatx16{};
    float m_run = -INFINITY, l_run = 0.f, l_exact = 0.f;
    floatx16 sacc[T::kKB];        // S^T of the tile between its S and sm phases
    V8 pf[T::kKB][2];         // P^T of the tile between its sm and PV phases
#pragma unroll
    for (int kb = 0; kb < T::kKB; ++kb) pf[kb][0] = pf[kb][1] = V8{};

    // ---- async tile copies (same chunk assignment as the kernel above)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t cp_koff[T::kLoadsPerWave], cp_voff[T::kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < T::kLoadsPerWave; ++i) {
        const int slot = (wave * T::kLoadsPerWave + i) * 64 + lane;
        const int r = slot / T::kCPR, p = slot % T::kCPR;
        cp_koff[i] = (uint32_t)(r * T::kRowBytes + 16 * (p ^ swz_k<D>(r)));
        cp_voff[i] = (uint32_t)(r * T::kRowBytes + 16 * (p ^ swz_v<D>(r)));
    }
    auto issue_copy = [&](const E* head, const uint32_t* cp_off, int kt, char* dst) {
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BN>(head, cp_off, wave_u, kv_t0 + kt, N, dst);
    };

    // ---- per-lane parts of the LDS fragment addresses
    int k_lane_off[T::kDS];
#pragma unroll
    for (int s = 0; s < T::kDS; ++s)
        k_lane_off[s] = l32 * T::kRowBytes + 16 * ((2 * s + h) ^ swz_k<D>(l32));
    const int vg = lane >> 4, vt = (lane >> 2) & 3, va = lane & 3;
    const int v_row_lane = 4 * (vg >> 1) + vt;
    int v_lane_off[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) {
        const int c = 4 * db + 2 * (vg & 1) + (va >> 1);
        v_lane_off[db] = v_row_lane * T::kRowBytes + 16 * (c ^ swz_v<D>(v_row_lane)) + 8 * (va & 1);
    }

    // ---- MFMA phase: PV(t-1) and S(t), interleaved so that consecutive
    // MFMAs never feed the same accumulator (4 O^T blocks + 2 S^T blocks).
    // Operand fragments are read from LDS two steps ahead of their MFMAs
    // (the scheduling fences keep the compiler from sinking the reads next
    // to their uses).  PV(-1) multiplies a zero P by a zero-filled V buffer;
    // the S(n_w) of a wave's last MFMA phase is computed and discarded, so
    // every phase runs the same straight-line code.  The phase also adds the
    // rounded weights of P(t-1) to l_run (two per v_dot2 against (1, 1)):
    // work taken out of the softmax phase, done while the partner wave
    // issues no MFMAs.  At D = 128 half of those sums run while the first
    // operand reads are in flight and half after the MFMAs; at D = 64 (a
    // phase of 16 MFMAs) all run after them.
    constexpr int kSteps = T::kDS * T::kKB;  // == number of PV MFMAs
    static_assert(kSteps == T::kKB * 2 * T::kDB, "one PV and one S MFMA per step");
    constexpr int kSumsFirst = D == 128 ? 1 : 0;  // halves ms of pf summed ahead of the MFMAs (bit ms)
    auto sum_rounded = [&](int halves) {
        if (halves == 0) return;
        float ls0 = l_run, ls1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                if (!((halves >> ms) & 1)) continue;
#pragma unroll
                for (int u = 0; u < 8; u += 2) {
                    const V2 pp = {pf[kb][ms][u], pf[kb][ms][u + 1]};
                    if ((u >> 1) & 1) ls1 = Half<E>::sum2(pp, ls1);
                    else ls0 = Half<E>::sum2(pp, ls0);
                }
            }
        l_run = ls0 + ls1;
    };
    auto read_v = [&](const char* vprev, int i) {
        const int step = i / T::kDB, db = i % T::kDB;
        const char* p0 = vprev + 16 * step * T::kRowBytes + v_lane_off[db];
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 8 * T::kRowBytes));
        return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto read_k = [&](const char* klds, int i) {
        const int s = i / T::kKB, kb = i % T::kKB;
        return *reinterpret_cast<const V8*>(klds + 32 * kb * T::kRowBytes + k_lane_off[s]);
    };
    auto mfma_phase = [&](int t, const char* klds, const char* vprev) {
        if (t > n_w) return;
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb) sacc[kb] = floatx16{};
        constexpr int kAhead = 2;
        V8 vr[kAhead + 1], kr[kAhead + 1];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
            vr[i] = read_v(vprev, i);
            kr[i] = read_k(klds, i);
        }
        if constexpr (kSumsFirst != 0) {
            __builtin_amdgcn_sched_barrier(0);
            sum_rounded(kSumsFirst);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            if (i + kAhead < kSteps) {
                vr[(i + kAhead) % (kAhead + 1)] = read_v(vprev, i + kAhead);
                kr[(i + kAhead) % (kAhead + 1)] = read_k(klds, i + kAhead);
            }
            __builtin_amdgcn_sched_barrier(0);
            {
                const int step = i / T::kDB, db = i % T::kDB;
                oacc[db] = Half<E>::mfma(vr[i % (kAhead + 1)], pf[step >> 1][step & 1],
                                                                   oacc[db]);
            }
            {
                const int s = i / T::kKB, kb = i % T::kKB;
                sacc[kb] = Half<E>::mfma(kr[i % (kAhead + 1)], qf[s], sacc[kb]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        sum_rounded(3 & ~kSumsFirst);
    };

    // ---- VALU phase: mask (boundary tiles), online softmax, rescale.
    // The weights are first taken against the running max as it stands,
    // P = exp2(s*c - m_run), with no max of the tile: the max only has to
    // move when some weight would leave the range of the 16-bit P (and of
    // fp32 O and l), and the lane's sum of P shows that after the fact: a
    // sum above Half<E>::kWeightSumCap (2^32 for bf16, 2^15 for fp16), an
    // inf, or the NaN of a row with no max yet fails the test.  Only then
    // is the tile's row max taken, O and l rescaled and P recomputed.  So
    // after a row's first tile the max moves only when its scores jump by
    // more than about 27 (bf16) or 10 (fp16) in log2 units, and the common
    // tile runs no max reduction ahead of its exponentials.  Large weights
    // lose nothing: fp32 O and l and the 16-bit P are relative formats, and
    // the weight of the key that last set the max was 1, so l >= 1 and tiny
    // weights stay negligible.  P is rounded once; l_exact sums the fp32
    // weights (for L), l_run the rounded ones (in the MFMA phase that
    // consumes P).
    // (in three fenced groups: all exponents, all exponentials, then the
    // rounding and the sums, so no consumer issues right behind the
    // transcendental it waits for)
    auto weights = [&](float m_sub) {
        float w[T::kKB][16];
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) w[kb][r] = fmaf(sacc[kb][r], c_log2, -m_sub);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) w[kb][r] = fast_exp2(w[kb][r]);
        __builtin_amdgcn_sched_barrier(0);
        float esum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int u = 0; u < 8; u += 2) {
                    const float p0 = w[kb][8 * ms + u], p1 = w[kb][8 * ms + u + 1];
                    const V2 pp = {(E)p0, (E)p1};
                    pf[kb][ms][u] = pp[0];
                    pf[kb][ms][u + 1] = pp[1];
                    esum[(u >> 1) & 3] += p0;
                    esum[((u >> 1) + 1) & 3] += p1;
                }
        return (esum[0] + esum[1]) + (esum[2] + esum[3]);
    };
    // The phase runs at raised wave priority: where the two waves of a SIMD
    // both have an instruction ready, the softmax's VALU issues ahead of the
    // partner's MFMA (the softmax phase is the longer one; -2 % at D = 64).
    auto valu_phase = [&](int t) {
        if (t < 0 || t >= n_w) return;
        if (MASK == kMaskLocal && t < w_first) {
            // a tile before the window of every row of the wave: P = 0, so
            // the PV product of the next MFMA phase adds nothing
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb) pf[kb][0] = pf[kb][1] = V8{};
            return;
        }
        __builtin_amdgcn_s_setprio(1);
        const int kbase = (kv_t0 + t) * BN;
        if (tile_needs_mask<MASK>(p, kbase, BN, N, qw0, qw1)) {
            __asm__ volatile("");  // keep this a branch, not a select per element
            // key kbase + 32 kb + acc_row(r, h) is visible iff its
            // compile-time part 32 kb + 8 (r / 4) + r % 4 lies in [lim_lo, lim]
            const int query = qw0 + l32;
            const int lim = key_hi<MASK>(p, query, N) - kbase - 4 * h;
            const int lim_lo = key_lo<MASK>(p, query) - kbase - 4 * h;
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int idx = 32 * kb + 8 * (r >> 2) + (r & 3);
                    if (idx > lim || (MASK == kMaskLocal && idx < lim_lo)) sacc[kb][r] = -INFINITY;
                }
        }
        float e_tile = weights(m_run);
        if (__any(!(e_tile <= Half<E>::kWeightSumCap))) {  // (not ">": NaN must fail too)
            __asm__ volatile("");
            // row max as four independent v_maximum3 chains, then a short tree
            float mxp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float& m4 = mxp[((kb * 16 + r) >> 1) & 3];
                    m4 = __builtin_elementwise_maximum(m4, __builtin_elementwise_maximum(sacc[kb][r], sacc[kb][r + 1]));
                }
            float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mxp[0], mxp[1]),
                                                     __builtin_elementwise_maximum(mxp[2], mxp[3]));
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            const float m_new = fmaxf(m_run, mx * c_log2);
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
            l_exact *= alpha;
#pragma unroll
            for (int db = 0; db < T::kDB; ++db) oacc[db] *= alpha;
            e_tile = weights(m_run == -INFINITY ? 0.f : m_run);
        }
        l_exact += e_tile;
        __builtin_amdgcn_s_setprio(0);
    };

    // ---- prologue: K_0 in buffer 0; V buffer 1 zeroed (read by PV(-1))
    for (int i = tid; i < T::kTileBytes / 16; i += T::kThreads)
        reinterpret_cast<uint4*>(sV1)[i] = make_uint4(0, 0, 0, 0);
    if (n_kv > 0) issue_copy(Kh, cp_koff, 0, sK0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- 2 n_kv + 2 periods, four per loop trip (two tiles)
    const int n_periods = 2 * n_kv + 2;
    for (int p0 = 0; p0 < n_periods; p0 += 4) {
        const int t0 = p0 >> 1;  // even tile of this trip
        // period p0: copies K_{t0+1} -> buf 1, V_{t0} -> buf 0.
        //            A: PV(t0-1) [V buf 1] + S(t0) [K buf 0];  B: sm(t0-1)
        if (t0 + 1 < n_kv) issue_copy(Kh, cp_koff, t0 + 1, sK1);
        if (t0 < n_kv) issue_copy(Vh, cp_voff, t0, sV0);
        if (grp == 0) mfma_phase(t0, sK0, sV1);
        else valu_phase(t0 - 1);
        // period p0+1: B: PV(t0-1) [V buf 1] + S(t0) [K buf 0];  A: sm(t0)
        if (grp == 1) mfma_phase(t0, sK0, sV1);
        else valu_phase(t0);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of K_{t0+1}, V_{t0}
        lds_barrier();
        // period p0+2: copies K_{t0+2} -> buf 0, V_{t0+1} -> buf 1.
        //              A: PV(t0) [V buf 0] + S(t0+1) [K buf 1];  B: sm(t0)
        if (t0 + 2 < n_kv) issue_copy(Kh, cp_koff, t0 + 2, sK0);
        if (t0 + 1 < n_kv) issue_copy(Vh, cp_voff, t0 + 1, sV1);
        if (grp == 0) mfma_phase(t0 + 1, sK1, sV0);
        else valu_phase(t0);
        // period p0+3: B: PV(t0) [V buf 0] + S(t0+1) [K buf 1];  A: sm(t0+1)
        if (grp == 1) mfma_phase(t0 + 1, sK1, sV0);
        else valu_phase(t0 + 1);
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();
    }

    // ---- epilogue: one normalisation, L = (m + log2 l) * ln 2, RNE store.
    // The rounded O goes through LDS (the wave's own 32 rows in a K/V buffer
    // the loop no longer reads) so that it leaves as whole rows, 16 bytes per
    // lane: a lane holds 4-value pieces of one row, and storing those
    // directly would touch 32 rows per instruction.
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
        const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const auto se = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_exact), __float_as_uint(l_exact), false, false);
        const float l_ex = __uint_as_float(se[0]) + __uint_as_float(se[1]);
        const int query = qw0 + l32;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const float lse = (m_run + fast_log2(l_ex)) * kLn2;
        if constexpr (SPLIT) {
            if (query < M) {
                float* orow = partial_row(p, task, query, D);
#pragma unroll
                for (int db = 0; db < T::kDB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const floatx4 x = {oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv,
                                           oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
                        *reinterpret_cast<floatx4*>(orow + 32 * db + 8 * g + 4 * h) = x;
                    }
                if (h == 0) *partial_l(p, task, query) = lse;
            }
        } else {
            // the wave's 32 rows x D, rows of kRowBytes whose 16-byte chunks
            // are XOR-swizzled by the row (conflict-free row reads, at most
            // two-way conflicts on the 8-byte writes)
            static_assert(32 * T::kRowBytes * 2 <= T::kTileBytes, "staging space");
            char* stage = (wave < 2 ? sK0 : wave < 4 ? sV0 : wave < 6 ? sK1 : sV1) + (wave & 1) * 32 * T::kRowBytes;
            const int rsw = l32 % T::kCPR;
#pragma unroll
            for (int db = 0; db < T::kDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = 4 * db + g;  // 16-byte chunk (8 values of d) of the row
                    const uint32_t w0 = pack2<E>(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
                    const uint32_t w1 = pack2<E>(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
                    *reinterpret_cast<uint2*>(stage + l32 * T::kRowBytes + 16 * (c ^ rsw) + 8 * h) = make_uint2(w0, w1);
                }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave reads back its own writes
            constexpr int kRowsPerRead = 64 / T::kCPR;
            const int rr = lane / T::kCPR, cc = lane % T::kCPR;
            E* const obase = O + (task.sv.q_row0 + qw0) * D;
#pragma unroll
            for (int i = 0; i < 32 / kRowsPerRead; ++i) {
                const int r = i * kRowsPerRead + rr;
                const uint4 x = *reinterpret_cast<const uint4*>(stage + r * T::kRowBytes + 16 * (cc ^ (r % T::kCPR)));
                if (qw0 + r < M) *reinterpret_cast<uint4*>(obase + (int64_t)r * D + 8 * cc) = x;
            }
            if (h == 0 && query < M) LSE[task.sv.q_row0 + query] = lse;
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel (v_mfma_f32_32x32x2_f32: true fp32 products, no reduced-precision
// shortcut)
// ---------------------------------------------------------------------------
// K and V tiles are copied global -> LDS by the load unit as in the 16-bit
// kernels (16 bytes per lane, no VGPR staging, unpadded rows whose 16-byte
// chunks are XOR-swizzled), which keeps the registers free for Q, O and S.
template <int D, int BN, int NW>
struct F32Traits {
    static constexpr int kThreads = NW * 64;
    static constexpr int kBM = 32 * NW;
    static constexpr int kKB = BN / 32;
    static constexpr int kDB = D / 32;
    static constexpr int kHalfD = D / 2;          // d values per lane half
    static constexpr int kRowBytes = D * 4;
    static constexpr int kCPR = D / 4;            // 16-byte chunks per row
    static constexpr int kTileBytes = BN * kRowBytes;
    static constexpr int kTileChunks = BN * kCPR;
    static constexpr int kLoadsPerWave = kTileChunks / (64 * NW);  // per tensor per tile
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(kTileChunks % (64 * NW) == 0, "loader split");
};

// Chunk XORs of the fp32 tiles.  K: a quarter-wave reads one logical chunk
// (4 floats of d) of 16 consecutive rows; XOR with the row's low 4 bits puts
// them in 16 distinct bank groups.  V: lanes 0-31 read 32 floats of d (8
// chunks) of key row r and lanes 32-63 the same d of row r + 4 (bit 2 of the
// row is the lane half); XOR 8 moves the second row's 8 chunks to the other
// half of the bank space.
__device__ __forceinline__ int swz_k_f32(int r) { return r & 15; }
__device__ __forceinline__ int swz_v_f32(int r) { return 8 * ((r >> 2) & 1); }

// Register budget: two waves per SIMD (as many as 64 KiB of LDS per
// workgroup allows), three for the 32-key tiles at D = 64 (32 KiB of LDS).
template <int D, int BN, int NW, int MASK, bool SPLIT>
__global__ void __launch_bounds__(NW * 64, (D == 64 && BN == 32) ? 3 : 2)
fa2_fwd_f32_kernel(const FwdParams p) {
    using T = F32Traits<D, BN, NW>;
    const float* __restrict__ Q = static_cast<const float*>(p.q);
    const float* __restrict__ K = static_cast<const float*>(p.k);
    const float* __restrict__ V = static_cast<const float*>(p.v);
    float* __restrict__ O = static_cast<float*>(p.o);
    float* __restrict__ LSE = p.lse;
    const float c_log2 = p.c_log2;
    __shared__ __attribute__((aligned(1024))) char sK0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sK1[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sV1[T::kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    const WgTask task = wg_task<MASK, SPLIT>(p, T::kBM, BN);
    const int M = task.sv.M, N = task.sv.N;
    const int qw0 = task.qt * T::kBM + wave * 32;
    const int qw1 = min(qw0 + 32, M) - 1;

    const float* Qh = Q + task.sv.q_row0 * D;
    const float* Kh = K + task.sv.kv_row0 * D;
    const float* Vh = V + task.sv.kv_row0 * D;

    // local tile kt is K/V tile kv_t0 + kt of the head
    const int kv_t0 = task.t_begin;
    const int n_kv = task.n_kv;
    const WaveRange wtiles = wave_tiles<MASK>(p, task, qw0, 32, BN);

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

    // ---- async tile copies: wave w moves chunks [w*L*64, (w+1)*L*64) of each
    // tensor's tile; LDS slot s holds row s / CPR, physical chunk s % CPR,
    // i.e. logical chunk (s % CPR) ^ swz(row).
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t cp_koff[T::kLoadsPerWave], cp_voff[T::kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < T::kLoadsPerWave; ++i) {
        const int slot = (wave * T::kLoadsPerWave + i) * 64 + lane;
        const int r = slot / T::kCPR, c = slot % T::kCPR;
        cp_koff[i] = (uint32_t)(r * T::kRowBytes + 16 * (c ^ swz_k_f32(r)));
        cp_voff[i] = (uint32_t)(r * T::kRowBytes + 16 * (c ^ swz_v_f32(r)));
    }
    auto issue_tile = [&](int kt, char* kdst, char* vdst) {
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BN>(Kh, cp_koff, wave_u, kv_t0 + kt, N, kdst);
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BN>(Vh, cp_voff, wave_u, kv_t0 + kt, N, vdst);
    };

    // per-lane parts of the LDS operand addresses: K row l32 (of each 32-row
    // block) at logical chunk h*D/8 + s/4; V element (row, d = 32 db + l32)
    // of rows whose bit 2 is h
    const int k_lane = l32 * T::kRowBytes;
    const int k_swz = swz_k_f32(l32);
    int v_lane_off[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db)
        v_lane_off[db] = 16 * ((8 * db + (l32 >> 2)) ^ (8 * h)) + 4 * (l32 & 3);

    // (always inlined: an out-of-line call would keep O, S and Q in memory)
    auto compute_tile = [&](int kt, const char* klds, const char* vlds) __attribute__((always_inline)) {
        floatx16 sacc[T::kKB];
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb) sacc[kb] = floatx16{};
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb) {
            const char* krow = klds + 32 * kb * T::kRowBytes + k_lane;
#pragma unroll
            for (int s = 0; s < T::kHalfD; s += 4) {
                const int c = h * (T::kHalfD / 4) + s / 4;
                const floatx4 kf = *reinterpret_cast<const floatx4*>(krow + 16 * (c ^ k_swz));
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[u], qf[s + u], sacc[kb], 0, 0, 0);
            }
        }
        // The softmax runs at raised wave priority: the three waves of a SIMD
        // come from three workgroups, and issuing a wave's softmax ahead of
        // the others' MFMAs gets its PV products and its workgroup's barrier
        // sooner (-1.3 % at D = 64, -7 % causal; +-0 at D = 128).
        __builtin_amdgcn_s_setprio(1);

        const int kbase = (kv_t0 + kt) * BN;
        if (tile_needs_mask<MASK>(p, kbase, BN, N, qw0, qw1)) {
            const int query = qw0 + l32;
            const int hi = key_hi<MASK>(p, query, N), lo = key_lo<MASK>(p, query);
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kbase + 32 * kb + acc_row(r, h);
                    if (key > hi || key < lo) sacc[kb][r] = -INFINITY;
                }
        }

        // Two ways to the weights.  Eager (the three-waves-per-SIMD form,
        // 32-key tiles at D = 64): the tile's row max first; the running max
        // moves (and O, l are rescaled) only when some row's max grew by more
        // than 8 in log2 units, so the weights stay below 2^8.  Lazy (every
        // other form): the weights are taken against the running max as it
        // stands, and only when a lane's sum leaves [0, 2^64] (a weight above
        // that, an inf, or the NaN of a row with no max yet) is the tile's
        // row max taken, O and l rescaled and the weights recomputed.  fp32
        // O and l hold weights up to 2^64 as accurately as weights up to 1
        // (relative formats; the key that last set the max has weight 1, so
        // l >= 1).  The lazy form keeps the weights beside the scores (16
        // more live registers), which at three waves per SIMD cost more than
        // the max it saves.
        constexpr bool kEagerMax = D == 64 && BN == 32;
        float lsum = -1.f;
        if constexpr (!kEagerMax) {
            auto weights = [&]() __attribute__((always_inline)) {
                float w[T::kKB][16];
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) w[kb][r] = fast_exp2(fmaf(sacc[kb][r], c_log2, -m_run));
                float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) l4[r & 3] += w[kb][r];
                const float e = (l4[0] + l4[1]) + (l4[2] + l4[3]);
                if (__any(!(e <= 0x1p64f))) return -1.f;  // (not ">": NaN must fail too)
#pragma unroll
                for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[kb][r] = w[kb][r];
                return e;
            };
            lsum = weights();
        }
        if (lsum < 0.f) {
            if constexpr (!kEagerMax) __asm__ volatile("");  // a rarely taken branch, not selects
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, xchg_half(mx));
            const float m_tile = mx * c_log2;
            if (!kEagerMax || __any(m_tile > m_run + 8.f)) {
                __asm__ volatile("");  // a rarely taken branch, not selects
                const float m_new = fmaxf(m_run, m_tile);
                const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) oacc[db] *= alpha;
            }
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
            lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pw = fast_exp2(fmaf(sacc[kb][r], c_log2, -m_use));
                    sacc[kb][r] = pw;
                    lsum += pw;
                }
        }
        l_run += lsum;
        __builtin_amdgcn_s_setprio(0);

        // O^T += V^T P^T: MFMA step r contracts key acc_row(r, h) in each half
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const char* vrow = vlds + (32 * kb + acc_row(r, 0)) * T::kRowBytes + 4 * h * T::kRowBytes;
#pragma unroll
                for (int db = 0; db < T::kDB; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        *reinterpret_cast<const float*>(vrow + v_lane_off[db]), sacc[kb][r], oacc[db], 0, 0, 0);
            }
    };

    // ---- main loop, unrolled by two over the buffer pair so that every LDS
    // access names its buffer (the copy in flight never aliases the one read)
    if (n_kv > 0) issue_tile(0, sK0, sV0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto run_tile = [&](int kt, const char* klds, const char* vlds) __attribute__((always_inline)) {
        if (kt >= wtiles.first && kt < wtiles.end) compute_tile(kt, klds, vlds);
    };
    for (int kt = 0; kt < n_kv; kt += 2) {
        if (kt + 1 < n_kv) issue_tile(kt + 1, sK1, sV1);
        run_tile(kt, sK0, sV0);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next tile have landed
        __syncthreads();
        if (kt + 1 >= n_kv) break;
        if (kt + 2 < n_kv) issue_tile(kt + 2, sK0, sV0);
        run_tile(kt + 1, sK1, sV1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    const float l_tot = l_run + xchg_half(l_run);
    const int query = qw0 + l32;
    if (query < M) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        // split K/V: the partial result goes to the workspace (also fp32)
        float* orow = SPLIT ? partial_row(p, task, query, D) : O + (task.sv.q_row0 + query) * D;
        float* lrow = SPLIT ? partial_l(p, task, query) : LSE + task.sv.q_row0 + query;
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
        if (h == 0) *lrow = (m_run + fast_log2(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// split K/V: combine the partial results
// ---------------------------------------------------------------------------
// Split s saw the keys of its range only and stored O_s = sum_j e_j v_j / l_s
// and L_s = log l_s with l_s = sum_j e_j, e_j = exp(score_j) over its visible
// keys.  The full row has l = sum_s l_s, so L = log sum_s exp(L_s) and
// O = sum_s exp(L_s - L) O_s exactly: the stored logsumexp is what makes the
// partials combinable ("FlashAttention-2 from PyTorch to Triton", the role of
// L; "From FlashAttention to FlashAttention 2", section "Layer 2", the
// split-K/V path of the dispatch).
// One wave per query row; each lane holds D / 64 consecutive values.  The
// split logsumexps are loaded at once (lane i holds splits i and i + 64),
// reduced across the wave, and the partial rows are then loaded eight splits
// at a time, so a row costs a few memory latencies, not one per split.
template <typename OutT, int D>
__global__ void __launch_bounds__(256)
fa2_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_l, OutT* __restrict__ O,
                 float* __restrict__ LSE, int rows, int n_splits) {
    constexpr int kPer = D / 64;
    static_assert(kPer == 1 || kPer == 2, "head dim");
    static_assert(FA2_MAX_SPLITS <= 128, "two splits per lane");
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // wave-uniform
    const float la = lane < n_splits ? ws_l[(int64_t)lane * rows + row] : -INFINITY;
    const float lb = lane + 64 < n_splits ? ws_l[(int64_t)(lane + 64) * rows + row] : -INFINITY;
    float m = fmaxf(la, lb);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    // weights exp(L_s - m); a split that saw no visible key (L_s = -inf) has
    // weight 0 and stored O_s = 0
    const float wa = m == -INFINITY ? 0.f : fast_exp2((la - m) * kLog2e);
    const float wb = m == -INFINITY ? 0.f : fast_exp2((lb - m) * kLog2e);
    float wsum = wa + wb;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
    float acc[kPer] = {};
    const float* base = ws_o + (int64_t)row * D + lane * kPer;
    const int64_t split_stride = (int64_t)rows * D;
    for (int s0 = 0; s0 < n_splits; s0 += 8) {
        float x[8][kPer];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = min(s0 + j, n_splits - 1);  // past the last split: re-read it, weight 0
            const float* src = base + s * split_stride;
            if constexpr (kPer == 2) {
                const float2 v = *reinterpret_cast<const float2*>(src);
                x[j][0] = v.x;
                x[j][1] = v.y;
            } else {
                x[j][0] = src[0];
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = s0 + j;  // uniform across the wave
            const float w_lane = s < 64 ? wa : wb;
            const float w = s < n_splits ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_lane), s & 63)) : 0.f;
#pragma unroll
            for (int i = 0; i < kPer; ++i) acc[i] = fmaf(w, x[j][i], acc[i]);
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    OutT* dst = O + (int64_t)row * D + lane * kPer;
#pragma unroll
    for (int i = 0; i < kPer; ++i) dst[i] = static_cast<OutT>(acc[i] * inv);  // bf16, fp16: nearest even
    if (lane == 0) LSE[row] = m == -INFINITY ? -INFINITY : m + fast_log2(wsum) * kLn2;
}

// ---------------------------------------------------------------------------
// host side: validation, dispatch table, launch
// ---------------------------------------------------------------------------
// Dispatch on (dtype, head dim, causal), as the pages' C++ entry point does
// with its dtype/head-dim/bool switches; each entry is one compiled kernel.
struct Entry {
    int dtype, D, causal;
    const void* kernel;        // whole key range, writes o and lse
    const void* kernel_split;  // one key range per split, writes the workspace
    int threads;
    int block_m;    // query rows per workgroup
    int block_n;    // keys per K/V tile
    int wg_per_cu;  // workgroups resident per CU (registers / LDS)
};

#define FWD_KERNEL(...) reinterpret_cast<const void*>(&__VA_ARGS__)
#define FWD_PAIR(name, ...) FWD_KERNEL(name<__VA_ARGS__, false>), FWD_KERNEL(name<__VA_ARGS__, true>)
const Entry kTable[] = {
    // bf16, fp16: the ping-pong kernel, 8 waves (two per SIMD) sharing each
    // 64-key K/V tile, 256 query rows per workgroup.  At D = 64 it measured 5 %
    // faster than the plain 8-wave kernel (128-key tiles) on the ragged
    // cross-attention workload; 128-key ping-pong tiles gained nothing there.
    {FA2_DTYPE_BF16, 64, 0, FWD_PAIR(fa2_fwd_half_pp_kernel, __bf16, 64, 64, kMaskNone), 512, 256, 64, 1},
    {FA2_DTYPE_BF16, 64, 1, FWD_PAIR(fa2_fwd_half_pp_kernel, __bf16, 64, 64, kMaskCausal), 512, 256, 64, 1},
    {FA2_DTYPE_BF16, 128, 0, FWD_PAIR(fa2_fwd_half_pp_kernel, __bf16, 128, 64, kMaskNone), 512, 256, 64, 1},
    {FA2_DTYPE_BF16, 128, 1, FWD_PAIR(fa2_fwd_half_pp_kernel, __bf16, 128, 64, kMaskCausal), 512, 256, 64, 1},
    {FA2_DTYPE_F16, 64, 0, FWD_PAIR(fa2_fwd_half_pp_kernel, _Float16, 64, 64, kMaskNone), 512, 256, 64, 1},
    {FA2_DTYPE_F16, 64, 1, FWD_PAIR(fa2_fwd_half_pp_kernel, _Float16, 64, 64, kMaskCausal), 512, 256, 64, 1},
    {FA2_DTYPE_F16, 128, 0, FWD_PAIR(fa2_fwd_half_pp_kernel, _Float16, 128, 64, kMaskNone), 512, 256, 64, 1},
    {FA2_DTYPE_F16, 128, 1, FWD_PAIR(fa2_fwd_half_pp_kernel, _Float16, 128, 64, kMaskCausal), 512, 256, 64, 1},
    // fp32: 4 waves, 128 query rows; at D = 64 non-causal 32-key tiles with
    // three workgroups per CU measured ~4 % faster than 64-key tiles with
    // two, and ~20 % slower under a causal mask (twice the masked diagonal
    // tiles and barriers), which keeps 64-key tiles
    {FA2_DTYPE_F32, 64, 0, FWD_PAIR(fa2_fwd_f32_kernel, 64, 32, 4, kMaskNone), 256, 128, 32, 3},
    {FA2_DTYPE_F32, 64, 1, FWD_PAIR(fa2_fwd_f32_kernel, 64, 64, 4, kMaskCausal), 256, 128, 64, 2},
    {FA2_DTYPE_F32, 128, 0, FWD_PAIR(fa2_fwd_f32_kernel, 128, 32, 4, kMaskNone), 256, 128, 32, 2},
    {FA2_DTYPE_F32, 128, 1, FWD_PAIR(fa2_fwd_f32_kernel, 128, 32, 4, kMaskCausal), 256, 128, 32, 2},
};
// Few query rows per (K/V) head -- decoding, where M is one token or a few
// per query head -- leave most of a 256-row workgroup empty, and the work is
// reading K and V once.  These entries take 64 rows per workgroup (two
// waves, one K/V tile double-buffered in 64 KiB of LDS, two workgroups per
// CU), so that the split count that fills the GPU spreads the keys over more
// workgroups and HBM, not the matrix core, sets the time.  (Their "two
// waves per SIMD" bound is not met -- they take 218-256 VGPRs and 96-142
// AGPRs -- and the compiler warns; LDS allows one wave per SIMD anyway.  A
// bound of one wave moved still more state into AGPRs, with copies.)
constexpr int64_t kShortRows = 64;  // rows per (K/V) head up to which kShortTable serves
const Entry kShortTable[] = {
    {FA2_DTYPE_BF16, 64, 0, FWD_PAIR(fa2_fwd_half_kernel, __bf16, 64, 128, 2, 1, 2, 2, kMaskNone), 128, 64, 128, 2},
    {FA2_DTYPE_BF16, 64, 1, FWD_PAIR(fa2_fwd_half_kernel, __bf16, 64, 128, 2, 1, 2, 2, kMaskCausal), 128, 64, 128, 2},
    {FA2_DTYPE_BF16, 128, 0, FWD_PAIR(fa2_fwd_half_kernel, __bf16, 128, 64, 2, 1, 2, 2, kMaskNone), 128, 64, 64, 2},
    {FA2_DTYPE_BF16, 128, 1, FWD_PAIR(fa2_fwd_half_kernel, __bf16, 128, 64, 2, 1, 2, 2, kMaskCausal), 128, 64, 64, 2},
    {FA2_DTYPE_F16, 64, 0, FWD_PAIR(fa2_fwd_half_kernel, _Float16, 64, 128, 2, 1, 2, 2, kMaskNone), 128, 64, 128, 2},
    {FA2_DTYPE_F16, 64, 1, FWD_PAIR(fa2_fwd_half_kernel, _Float16, 64, 128, 2, 1, 2, 2, kMaskCausal), 128, 64, 128, 2},
    {FA2_DTYPE_F16, 128, 0, FWD_PAIR(fa2_fwd_half_kernel, _Float16, 128, 64, 2, 1, 2, 2, kMaskNone), 128, 64, 64, 2},
    {FA2_DTYPE_F16, 128, 1, FWD_PAIR(fa2_fwd_half_kernel, _Float16, 128, 64, 2, 1, 2, 2, kMaskCausal), 128, 64, 64, 2},
};
// The same decode form with 32-key tiles in a ring of four buffer pairs
// (three tiles' copies in flight) for D = 128 without a mask, taken when each
// split covers at least kLongSplitKeys keys: at 16 splits over 16384 keys it
// measured 6 % faster than the double-buffered 64-key form, and 1.4-3.5 %
// slower at 512 and 256 keys per split, where a split's two 32-key chains
// per 64 keys outweigh the deeper prefetch.
constexpr int64_t kLongSplitKeys = 1024;
const Entry kShortLongTable[] = {
    {FA2_DTYPE_BF16, 128, 0, FWD_PAIR(fa2_fwd_half_kernel, __bf16, 128, 32, 2, 1, 2, 4, kMaskNone), 128, 64, 32, 2},
    {FA2_DTYPE_F16, 128, 0, FWD_PAIR(fa2_fwd_half_kernel, _Float16, 128, 32, 2, 1, 2, 4, kMaskNone), 128, 64, 32, 2},
};
#undef FWD_PAIR

struct MergeEntry {
    int dtype, D;
    const void* kernel;
};
const MergeEntry kMergeTable[] = {
    {FA2_DTYPE_BF16, 64, FWD_KERNEL(fa2_merge_kernel<__bf16, 64>)},
    {FA2_DTYPE_BF16, 128, FWD_KERNEL(fa2_merge_kernel<__bf16, 128>)},
    {FA2_DTYPE_F16, 64, FWD_KERNEL(fa2_merge_kernel<_Float16, 64>)},
    {FA2_DTYPE_F16, 128, FWD_KERNEL(fa2_merge_kernel<_Float16, 128>)},
    {FA2_DTYPE_F32, 64, FWD_KERNEL(fa2_merge_kernel<float, 64>)},
    {FA2_DTYPE_F32, 128, FWD_KERNEL(fa2_merge_kernel<float, 128>)},
};

constexpr int kCUs = 256;  // MI355X; the split heuristic's design point

// Kernel for (dtype, D, causal) at `rows` query rows per head of the kernel
// view (the grouped rows of a K/V head when they are packed).
const Entry* find_entry(int dtype, int64_t D, int causal, int64_t rows) {
    if (rows <= kShortRows)
        for (const Entry& t : kShortTable)
            if (t.dtype == dtype && t.D == D && t.causal == causal) return &t;
    for (const Entry& t : kTable)
        if (t.dtype == dtype && t.D == D && t.causal == causal) return &t;
    return nullptr;
}


// The ring form of a decode entry when its splits are long enough (same
// rows per workgroup and workgroups per CU, so the split count stands).
const Entry* long_split_entry(const Entry* e, int64_t N, int splits) {
    if (e->block_m > kShortRows || N / splits < kLongSplitKeys) return e;
    for (const Entry& t : kShortLongTable)
        if (t.dtype == e->dtype && t.D == e->D && t.causal == e->causal) return &t;
    return e;
}

// Split count that fills the GPU: 1 when the unsplit grid already occupies
// three quarters of the workgroup slots; otherwise enough splits to fill them,
// with at least two K/V tiles per split.
int choose_splits(const Entry& e, int64_t BH, int64_t M, int64_t N) {
    const int64_t base = BH * ceil_div(M, e.block_m);
    const int64_t slots = (int64_t)kCUs * e.wg_per_cu;
    if (base <= 0 || base * 4 >= slots * 3) return 1;
    int64_t s = ceil_div(slots, base);
    s = std::min<int64_t>(s, std::max<int64_t>(1, ceil_div(N, e.block_n) / 2));
    s = std::min<int64_t>(s, FA2_MAX_SPLITS);
    return (int)std::max<int64_t>(1, s);
}

// Sliding-window and packed-sequence entry points: the ping-pong 16-bit
// kernel and the fp32 kernel, one instantiation per mask kind, unsplit.
struct LocalEntry {
    int dtype, D, mask, packed;  // packed: fa2_fwd_varlen's packed layout
    const void* kernel;
    int threads;
    int block_m;  // query rows per workgroup
};
#define LOCAL_HALF(E, code, mask)                                                                      \
    {code, 64, mask, 0, FWD_KERNEL(fa2_fwd_half_pp_kernel<E, 64, 64, mask, false>), 512, 256},         \
    {code, 128, mask, 0, FWD_KERNEL(fa2_fwd_half_pp_kernel<E, 128, 64, mask, false>), 512, 256},       \
    {code, 64, mask, 1, FWD_KERNEL(fa2_fwd_half_pp_kernel<E, 64, 64, mask, false, true>), 512, 256},   \
    {code, 128, mask, 1, FWD_KERNEL(fa2_fwd_half_pp_kernel<E, 128, 64, mask, false, true>), 512, 256}
#define LOCAL_F32(mask)                                                                                \
    {FA2_DTYPE_F32, 64, mask, 0, FWD_KERNEL(fa2_fwd_f32_kernel<64, 64, 4, mask, false>), 256, 128},     \
    {FA2_DTYPE_F32, 128, mask, 0, FWD_KERNEL(fa2_fwd_f32_kernel<128, 32, 4, mask, false>), 256, 128},   \
    {FA2_DTYPE_F32, 64, mask, 1, FWD_KERNEL(fa2_fwd_f32_kernel<64, 64, 4, mask, false>), 256, 128},     \
    {FA2_DTYPE_F32, 128, mask, 1, FWD_KERNEL(fa2_fwd_f32_kernel<128, 32, 4, mask, false>), 256, 128}
const LocalEntry kLocalTable[] = {
    LOCAL_HALF(__bf16, FA2_DTYPE_BF16, kMaskNone),  LOCAL_HALF(__bf16, FA2_DTYPE_BF16, kMaskCausal),
    LOCAL_HALF(__bf16, FA2_DTYPE_BF16, kMaskLocal), LOCAL_HALF(_Float16, FA2_DTYPE_F16, kMaskNone),
    LOCAL_HALF(_Float16, FA2_DTYPE_F16, kMaskCausal), LOCAL_HALF(_Float16, FA2_DTYPE_F16, kMaskLocal),
    LOCAL_F32(kMaskNone), LOCAL_F32(kMaskCausal), LOCAL_F32(kMaskLocal),
};
#undef LOCAL_HALF
#undef LOCAL_F32

const LocalEntry* find_local_entry(int dtype, int64_t D, int mask, int packed) {
    for (const LocalEntry& t : kLocalTable)
        if (t.dtype == dtype && t.D == D && t.mask == mask && t.packed == packed) return &t;
    return nullptr;
}

#undef FWD_KERNEL

int64_t workspace_bytes(int64_t BH, int64_t M, int64_t D, int n_splits) {
    if (n_splits <= 1) return 0;
    const int64_t rows = (int64_t)n_splits * BH * M;
    return ceil_div(rows * D * 4, 256) * 256 + rows * 4;
}

}  // namespace

extern "C" int64_t fa2_fwd_workspace_bytes(int64_t B, int64_t H, int64_t M, int64_t D, int n_splits) {
    if (B < 0 || H < 0 || M < 0 || D <= 0 || n_splits < 1 || n_splits > FA2_MAX_SPLITS) return -1;
    if (B > ((int64_t)1 << 31) || H > ((int64_t)1 << 31) || M > ((int64_t)1 << 31) || D > 4096) return -1;
    return workspace_bytes(B * H, M, D, n_splits);
}

extern "C" int fa2_fwd_num_splits(int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D, int causal,
                                  int dtype) {
    if (B < 0 || H < 0 || Hk < 1 || M < 0 || N <= 0) return 1;
    if (H > 0 && (Hk > H || H % Hk != 0)) return 1;
    if (B > ((int64_t)1 << 31) || H > ((int64_t)1 << 31) || M > ((int64_t)1 << 31)) return 1;
    const KernelShape ks = kernel_shape(B, H, Hk, M, causal);
    const Entry* e = find_entry(dtype, D, causal, ks.M);
    if (!e) return 1;
    return choose_splits(*e, ks.BH, ks.M, N);
}

// Split-K/V partials for callers that cannot allocate (fa2_fwd_ex_noalloc):
// one array per device, kept until the process ends.  Its name is a host-side
// stand-in; host code only ever uses the device address that
// hipGetSymbolAddress returns for it (scratch_address).
static __device__ __align__(256) char scratch[FA2_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's `scratch` array, looked up once per
// device (with that device current) and kept; FA2_OK or the failure status.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return launch_status(err);
    if (dev < 0 || dev >= kMaxDevices) return FA2_ERR_NO_DEVICE;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (err != hipSuccess || p == nullptr) return err != hipSuccess ? launch_status(err) : FA2_ERR_LAUNCH;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return FA2_OK;
}

// fa2_fwd_ex, with the split workspace either the caller's or (use_scratch)
// the device's static scratch array.
int fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
           float scale, int causal, int dtype, int n_splits,
           void* workspace, int64_t workspace_size, bool use_scratch, void* stream) {
    // ---- argument checks, all before any HIP call
    if (B < 0 || H < 0 || Hk < 1 || M < 0 || N <= 0 || D <= 0) return FA2_ERR_INVALID_ARGUMENT;
    // a pointer may be null only when its buffer holds no element
    const bool q_rows = B > 0 && H > 0 && M > 0, kv_rows = B > 0;
    if ((q_rows && (!q || !o || !lse)) || (kv_rows && (!k || !v))) return FA2_ERR_INVALID_ARGUMENT;
    if (H > 0 && (Hk > H || H % Hk != 0)) return FA2_ERR_INVALID_ARGUMENT;
    if (dtype != FA2_DTYPE_F32 && dtype != FA2_DTYPE_BF16 && dtype != FA2_DTYPE_F16) return FA2_ERR_INVALID_ARGUMENT;
    if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARGUMENT;
    if (!(scale > 0.f) || !isfinite(scale)) return FA2_ERR_INVALID_ARGUMENT;
    if (n_splits < 0 || n_splits > FA2_MAX_SPLITS) return FA2_ERR_INVALID_ARGUMENT;
    if (workspace_size < 0) return FA2_ERR_INVALID_ARGUMENT;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(lse, 4))
        return FA2_ERR_INVALID_ARGUMENT;

    if (!find_entry(dtype, D, causal, kShortRows + 1)) return FA2_ERR_UNSUPPORTED;

    // sizes: per-head offsets are 32-bit in the kernels, the grid is 1-D
    const int64_t kMax = (int64_t)1 << 31;
    if (B > kMax || H > kMax || M >= kMax || N >= kMax) return FA2_ERR_UNSUPPORTED;
    const int64_t BH = B * H;
    if (M * D >= kMax || N * D >= kMax || BH >= kMax) return FA2_ERR_UNSUPPORTED;
    const KernelShape ks = kernel_shape(B, H, Hk, M, causal);
    if (ks.M * D >= kMax) return FA2_ERR_UNSUPPORTED;
    const Entry* e = find_entry(dtype, D, causal, ks.M);
    // every forward kernel copies one head's K (V) tiles through a buffer
    // resource whose byte size, and the tile offsets inside it, are 32-bit
    const int64_t elt = dtype == FA2_DTYPE_F32 ? 4 : 2;
    if (N * D * elt >= kMax || ks.M * D * elt >= kMax) return FA2_ERR_UNSUPPORTED;
    const int splits = n_splits == 0 ? choose_splits(*e, ks.BH, ks.M, N) : n_splits;
    e = long_split_entry(e, N, splits);
    const int64_t n_qt = ceil_div(ks.M, e->block_m);
    if (n_qt * ks.BH * splits >= kMax) return FA2_ERR_UNSUPPORTED;

    const size_t o_bytes = (size_t)BH * M * D * elt;
    const size_t kv_bytes = (size_t)B * Hk * N * D * elt;
    const size_t lse_bytes = (size_t)BH * M * 4;
    if (overlaps(o, o_bytes, q, o_bytes) || overlaps(o, o_bytes, k, kv_bytes) ||
        overlaps(o, o_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, q, o_bytes) ||
        overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes) ||
        overlaps(lse, lse_bytes, o, o_bytes))
        return FA2_ERR_INVALID_ARGUMENT;
    const int64_t ws_need = workspace_bytes(BH, M, D, splits);
    if (use_scratch) {
        if (ws_need > FA2_NOALLOC_SCRATCH_BYTES) return FA2_ERR_SCRATCH;
    } else if (ws_need > 0) {
        if (!workspace || workspace_size < ws_need || misaligned(workspace, 16))
            return FA2_ERR_INVALID_ARGUMENT;
        const size_t w = (size_t)ws_need;
        if (overlaps(workspace, w, q, o_bytes) || overlaps(workspace, w, k, kv_bytes) ||
            overlaps(workspace, w, v, kv_bytes) || overlaps(workspace, w, o, o_bytes) ||
            overlaps(workspace, w, lse, lse_bytes))
            return FA2_ERR_INVALID_ARGUMENT;
    }

    if (M == 0 || BH == 0) return FA2_OK;
    if (use_scratch && ws_need > 0) {
        const int st = scratch_address(&workspace);
        if (st != FA2_OK) return st;
    }

    FwdParams prm{};  // dense layout, no window: cu_q = cu_k = null
    prm.q = q; prm.k = k; prm.v = v; prm.o = o; prm.lse = lse;
    prm.BH = (int)ks.BH; prm.H = (int)ks.H; prm.G = (int)ks.G;
    prm.Hk = (int)(ks.H / ks.G);
    prm.wl = prm.wr = -1;
    prm.M = (int)ks.M; prm.N = (int)N;
    prm.n_qt = (int)n_qt;
    prm.c_log2 = scale * 1.44269504088896340736f;  // scale * log2(e)
    const int64_t n_tiles = ceil_div(N, e->block_n);
    if (splits > 1) {
        prm.ws_o = static_cast<float*>(workspace);
        prm.ws_l = reinterpret_cast<float*>(static_cast<char*>(workspace) + ceil_div(splits * BH * M * D * 4, 256) * 256);
        prm.tiles_per_split = (int)ceil_div(n_tiles, splits);
    } else {
        prm.ws_o = prm.ws_l = nullptr;
        prm.tiles_per_split = (int)n_tiles;
    }

    hipStream_t st = static_cast<hipStream_t>(stream);
    void* args[] = {&prm};
    hipError_t err = hipLaunchKernel(splits > 1 ? e->kernel_split : e->kernel, dim3((unsigned)(n_qt * ks.BH * splits)),
                                     dim3(e->threads), args, 0, st);
    if (err == hipSuccess && splits > 1) {
        const MergeEntry* me = nullptr;
        for (const MergeEntry& t : kMergeTable)
            if (t.dtype == dtype && t.D == D) me = &t;
        if (!me) return FA2_ERR_UNSUPPORTED;  // unreachable: every forward entry has a merge
        const float* ws_o = prm.ws_o;
        const float* ws_l = prm.ws_l;
        int rows = (int)(BH * M), ns = splits;
        void* margs[] = {(void*)&ws_o, (void*)&ws_l, &o, &lse, &rows, &ns};
        err = hipLaunchKernel(me->kernel, dim3((unsigned)ceil_div(rows, 4)), dim3(256), margs, 0, st);
    }
    return launch_status(err);
}

}  // namespace

extern "C" int fa2_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
                          float scale, int causal, int dtype, int n_splits,
                          void* workspace, int64_t workspace_size, void* stream) {
    return fwd_ex(q, k, v, o, lse, B, H, Hk, M, N, D, scale, causal, dtype, n_splits, workspace,
                  workspace_size, false, stream);
}

extern "C" int fa2_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
                                  float scale, int causal, int dtype, int n_splits, void* stream) {
    return fwd_ex(q, k, v, o, lse, B, H, Hk, M, N, D, scale, causal, dtype, n_splits, nullptr, 0, true,
                  stream);
}

extern "C" int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t M, int64_t N, int64_t D,
                       float scale, int causal, int dtype, void* stream) {
    return fa2_fwd_ex(q, k, v, o, lse, B, H, H > 0 ? H : 1, M, N, D, scale, causal, dtype, 1, nullptr, 0,
                      stream);
}

extern "C" int fa2_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
                             float scale, int causal, int64_t window_left, int64_t window_right,
                             int dtype, void* stream) {
    // ---- argument checks, all before any HIP call
    if (B < 0 || H < 0 || Hk < 1 || M < 0 || N <= 0 || D <= 0) return FA2_ERR_INVALID_ARGUMENT;
    const bool q_rows = B > 0 && H > 0 && M > 0, kv_rows = B > 0;
    if ((q_rows && (!q || !o || !lse)) || (kv_rows && (!k || !v))) return FA2_ERR_INVALID_ARGUMENT;
    if (H > 0 && (Hk > H || H % Hk != 0)) return FA2_ERR_INVALID_ARGUMENT;
    if (dtype != FA2_DTYPE_F32 && dtype != FA2_DTYPE_BF16 && dtype != FA2_DTYPE_F16) return FA2_ERR_INVALID_ARGUMENT;
    if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARGUMENT;
    if (!(scale > 0.f) || !isfinite(scale)) return FA2_ERR_INVALID_ARGUMENT;
    if (window_left < -1 || window_right < -1) return FA2_ERR_INVALID_ARGUMENT;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(lse, 4))
        return FA2_ERR_INVALID_ARGUMENT;
    if (D != 64 && D != 128) return FA2_ERR_UNSUPPORTED;
    const int64_t kMax = (int64_t)1 << 31;
    if (B > kMax || H > kMax || M >= kMax || N >= kMax) return FA2_ERR_UNSUPPORTED;
    const int64_t BH = B * H;
    const size_t elt = dtype == FA2_DTYPE_F32 ? 4 : 2;
    if (M * D * (int64_t)elt >= kMax || N * D * (int64_t)elt >= kMax || BH >= kMax) return FA2_ERR_UNSUPPORTED;
    const size_t o_bytes = (size_t)BH * M * D * elt;
    const size_t kv_bytes = (size_t)B * Hk * N * D * elt;
    const size_t lse_bytes = (size_t)BH * M * 4;
    if (overlaps(o, o_bytes, q, o_bytes) || overlaps(o, o_bytes, k, kv_bytes) ||
        overlaps(o, o_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, q, o_bytes) ||
        overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes) ||
        overlaps(lse, lse_bytes, o, o_bytes))
        return FA2_ERR_INVALID_ARGUMENT;
    int64_t wl = window_left, wr = window_right;
    const int mask = normalise_window(wl, wr, causal, M, N);
    const LocalEntry* e = find_local_entry(dtype, D, mask, 0);
    if (!e) return FA2_ERR_UNSUPPORTED;
    const int64_t n_qt = ceil_div(M, e->block_m);
    if (n_qt * BH >= kMax) return FA2_ERR_UNSUPPORTED;
    if (M == 0 || BH == 0) return FA2_OK;

    FwdParams prm{};
    prm.q = q; prm.k = k; prm.v = v; prm.o = o; prm.lse = lse;
    prm.BH = (int)BH; prm.H = (int)H; prm.Hk = (int)Hk; prm.G = (int)(H / Hk);
    prm.M = (int)M; prm.N = (int)N;
    prm.n_qt = (int)n_qt;
    prm.tiles_per_split = (int)N;  // at least every tile
    prm.wl = (int)wl; prm.wr = (int)wr;
    prm.c_log2 = scale * kLog2e;
    void* args[] = {&prm};
    const hipError_t err = hipLaunchKernel(e->kernel, dim3((unsigned)(n_qt * BH)), dim3(e->threads), args, 0,
                                           static_cast<hipStream_t>(stream));
    return launch_status(err);
}

extern "C" int fa2_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int64_t B, int64_t H, int64_t Hk, int64_t total_q, int64_t total_k,
                              int64_t max_seqlen_q, int64_t D, float scale, int causal,
                              int64_t window_left, int64_t window_right, int dtype, void* stream) {
    // ---- argument checks, all before any HIP call
    if (B < 0 || H < 0 || Hk < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || D <= 0)
        return FA2_ERR_INVALID_ARGUMENT;
    if (max_seqlen_q > total_q) return FA2_ERR_INVALID_ARGUMENT;
    if (B > 0 && (!cu_seqlens_q || !cu_seqlens_k)) return FA2_ERR_INVALID_ARGUMENT;
    if ((H > 0 && total_q > 0 && (!q || !o || !lse)) || (total_k > 0 && (!k || !v))) return FA2_ERR_INVALID_ARGUMENT;
    if (H > 0 && (Hk > H || H % Hk != 0)) return FA2_ERR_INVALID_ARGUMENT;
    if (dtype != FA2_DTYPE_F32 && dtype != FA2_DTYPE_BF16 && dtype != FA2_DTYPE_F16) return FA2_ERR_INVALID_ARGUMENT;
    if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARGUMENT;
    if (!(scale > 0.f) || !isfinite(scale)) return FA2_ERR_INVALID_ARGUMENT;
    if (window_left < -1 || window_right < -1) return FA2_ERR_INVALID_ARGUMENT;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(lse, 4) ||
        misaligned(cu_seqlens_q, 4) || misaligned(cu_seqlens_k, 4))
        return FA2_ERR_INVALID_ARGUMENT;
    if (D != 64 && D != 128) return FA2_ERR_UNSUPPORTED;
    const int64_t kMax = (int64_t)1 << 31;
    const size_t elt = dtype == FA2_DTYPE_F32 ? 4 : 2;
    if (B >= kMax || H >= kMax || Hk >= kMax || total_q * D * (int64_t)elt >= kMax ||
        total_k * D * (int64_t)elt >= kMax)
        return FA2_ERR_UNSUPPORTED;
    const size_t o_bytes = (size_t)H * total_q * D * elt;
    const size_t kv_bytes = (size_t)Hk * total_k * D * elt;
    const size_t lse_bytes = (size_t)H * total_q * 4;
    if (overlaps(o, o_bytes, q, o_bytes) || overlaps(o, o_bytes, k, kv_bytes) ||
        overlaps(o, o_bytes, v, kv_bytes) || overlaps(lse, lse_bytes, q, o_bytes) ||
        overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes) ||
        overlaps(lse, lse_bytes, o, o_bytes))
        return FA2_ERR_INVALID_ARGUMENT;
    int64_t wl = window_left, wr = window_right;
    const int mask = normalise_window(wl, wr, causal, total_q, total_k);
    const LocalEntry* e = find_local_entry(dtype, D, mask, 1);
    if (!e) return FA2_ERR_UNSUPPORTED;
    const int64_t BH = B * H;
    const int64_t n_qt = ceil_div(max_seqlen_q, e->block_m);
    if (BH >= kMax || n_qt * BH >= kMax) return FA2_ERR_UNSUPPORTED;
    if (BH == 0 || n_qt == 0) return FA2_OK;

    FwdParams prm{};
    prm.q = q; prm.k = k; prm.v = v; prm.o = o; prm.lse = lse;
    prm.cu_q = cu_seqlens_q; prm.cu_k = cu_seqlens_k;
    prm.total_q = (int)total_q; prm.total_k = (int)total_k;
    prm.BH = (int)BH; prm.H = (int)H; prm.Hk = (int)Hk; prm.G = (int)(H / Hk);
    prm.n_qt = (int)n_qt;
    prm.tiles_per_split = (int)total_k + 1;  // at least every tile
    prm.wl = (int)wl; prm.wr = (int)wr;
    prm.c_log2 = scale * kLog2e;
    void* args[] = {&prm};
    const hipError_t err = hipLaunchKernel(e->kernel, dim3((unsigned)(n_qt * BH)), dim3(e->threads), args, 0,
                                           static_cast<hipStream_t>(stream));
    return launch_status(err);
}

extern "C" const char* fa2_status_string(int status) {
    switch (status) {
        case FA2_OK: return "FA2_OK: success";
        case FA2_ERR_INVALID_ARGUMENT: return "FA2_ERR_INVALID_ARGUMENT: null, misaligned or overlapping pointer, or bad size, dtype, causal flag or scale";
        case FA2_ERR_UNSUPPORTED: return "FA2_ERR_UNSUPPORTED: head dimension or problem size not supported by this build";
        case FA2_ERR_LAUNCH: return "FA2_ERR_LAUNCH: the HIP runtime rejected the kernel launch";
        case FA2_ERR_NO_DEVICE: return "FA2_ERR_NO_DEVICE: no usable gfx950 device";
        case FA2_ERR_SCRATCH: return "FA2_ERR_SCRATCH: the split partials need more than the static scratch array (FA2_NOALLOC_SCRATCH_BYTES) holds";
        default: return "unknown fa2 status";
    }
}
