// fa2_bwd.hip -- gradients of exact attention (the FlashAttention-2 backward
// schedule) for AMD CDNA4 / gfx950, behind the C ABI declared in include/fa2.h.
//
// What is computed, for the forward O = softmax(scale * Q K^T) V (optionally
// causal) whose per-row logsumexp L the forward pass stored, and an upstream
// gradient dO:
//
//   P     = exp(scale * Q K^T - L)              (recomputed, never stored)
//   dV    = P^T dO
//   dP    = dO V^T
//   Delta = rowsum(dO o O)                      (= rowsum(P o dP))
//   dS    = P o (dP - Delta)
//   dQ    = scale * dS K
//   dK    = scale * dS^T Q
//
// with dK, dV summed over the query heads that share a K/V head.  Sources:
// "From FlashAttention to FlashAttention 2", section "Layer 7: The Backward
// Kernel" (the recomputation of P from the stored L, the five products and
// the per-row correction term rowsum(dO o O)) and section "Backward Pass:
// Recomputation" (why only L is kept from the forward); "FlashAttention-2
// from PyTorch to Triton", opening section (L is the second output of the
// forward, stored for the backward).
//
// Schedule (our own design for gfx950):
//  * Delta per query row: the 16-bit dQ kernel computes it from the dO
//    fragments it holds anyway and one read of O, and stores it for the
//    dK/dV kernel, which runs after it; fp32 inputs use a small HBM-bound
//    kernel (one pass over O and dO) ahead of the other two;
//  * the dK/dV kernel gives each workgroup one tile of keys (32 per wave) of
//    one K/V head and streams the query tiles of every query head of its
//    group through LDS; K and V of the wave's keys stay in VGPRs (at
//    D = 128 in LDS instead, with two waves per 32 keys: the wave-pair
//    kernel), dK and dV accumulate in registers and are written once -- no
//    atomics;
//  * the dQ kernel gives each workgroup one tile of queries (32 per wave),
//    keeps Q and dO in VGPRs and streams K/V tiles through LDS, exactly like
//    the forward; it recomputes P and dP rather than accumulating dQ with
//    atomics from the dK/dV kernel, so every gradient is written once by one
//    workgroup and the result is deterministic run to run.
//
// MFMA operand mapping (32x32x16, bf16 / fp16; lane l owns accumulator column
// l % 32).  dK/dV kernel: S = Q K^T and dP = dO V^T take the tile's Q / dO
// rows as A operands (row reads from LDS) and the wave's K / V rows as B
// operands (registers), so each lane owns one key and holds 16 of the tile's
// queries; the P and dS accumulators are then exactly the B operands of
// dV^T += dO^T P and dK^T += Q^T dS, whose A operands are dO^T / Q^T read
// with ds_read_b64_tr_b16 in the matching query order.  dQ kernel: the
// forward's mapping (lane = query): S^T = K Q^T, dP^T = V dO^T, and
// dQ^T += K^T dS^T with K^T read transposed.  Q and dO tiles (dK/dV kernel)
// and K tiles (dQ kernel) are read both row-wise and transposed, so they use
// one XOR swizzle that keeps both patterns free of LDS bank conflicts.
// fp32 inputs run the same schedule on v_mfma_f32_32x32x2_f32 with P and dS
// kept in fp32 (the fp32 section below).

#include <hip/hip_runtime.h>
#include <math.h>
#include <limits.h>
#include <stdint.h>

#include <algorithm>

#include "fa2.h"
#include "fa2_common.h"

namespace {

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const void* o;      // the forward's output (16-bit paths: read by the dQ kernel for Delta)
    const float* lse;
    float* delta;       // written by the Delta pass, read by the dK/dV kernel
    void* dq;
    void* dk;
    void* dv;
    const int* cu_q;    // packed sequences: query row offsets [B + 1] (device), else null
    const int* cu_k;    // packed sequences: key row offsets [B + 1]
    int total_q, total_k;  // packed sequences: rows per head of q (o, dout, lse, delta) and of k (v)
    int BH;     // batch * query heads, as the kernels see them
    int BHk;    // batch * K/V heads
    int H, Hk;  // query and K/V heads, as the kernels see them
    int G;      // query heads per K/V head, as the kernels see them (0: none)
    int M, N;   // dense: query rows per head (kernel view), keys per head
    int n_qt;   // query tiles per head, of the kernel's own tile height
    int wl, wr; // sliding window: keys i - wl .. i + wr (-1: unbounded side)
    float c_log2;  // scale * log2(e)
    float scale;
};

// The sequence of batch b: the whole head in the dense layout (cu_q null),
// else rows cu_q[b] .. cu_q[b + 1] - 1 (keys cu_k[b] .. cu_k[b + 1] - 1) of
// each head of the packed layout, clamped into [0, total].
struct BwdSeq {
    int q0, k0;  // first query / key row of the sequence inside a head's rows
    int M, N;    // its query rows and keys
};
__device__ __forceinline__ BwdSeq bwd_seq(const BwdParams& p, int b) {
    BwdSeq s;
    if (p.cu_q == nullptr) {
        s.q0 = s.k0 = 0;
        s.M = p.M;
        s.N = p.N;
        return s;
    }
    const int q0 = min(max(p.cu_q[b], 0), p.total_q), q1 = min(max(p.cu_q[b + 1], q0), p.total_q);
    const int k0 = min(max(p.cu_k[b], 0), p.total_k), k1 = min(max(p.cu_k[b + 1], k0), p.total_k);
    s.q0 = q0;
    s.k0 = k0;
    s.M = q1 - q0;
    s.N = k1 - k0;
    return s;
}
// Row (of D elements) of q, o, dout, dq, lse, delta holding query row 0 of
// head bh's sequence, and of k, v, dk, dv holding key row 0 of K/V head bkv's.
__device__ __forceinline__ int64_t q_row0(const BwdParams& p, const BwdSeq& s, int bh) {
    return p.cu_q ? (int64_t)(bh % p.H) * p.total_q + s.q0 : (int64_t)bh * p.M;
}
__device__ __forceinline__ int64_t kv_row0(const BwdParams& p, const BwdSeq& s, int bkv) {
    return p.cu_q ? (int64_t)(bkv % p.Hk) * p.total_k + s.k0 : (int64_t)bkv * p.N;
}

// The stored logsumexp of a row in log2 units, as the exponent offset of
// P = exp2(S c - L2).  A row that saw no key (L = -inf: possible under a
// window, or for a packed sequence without keys) has no gradient; +inf makes
// its P exactly 0 whatever its (masked, -inf) scores, where -inf would give
// exp2(-inf + inf) = NaN.  Rows past M pass +inf too.
__device__ __forceinline__ float l2_of(float lse) {
    return lse == -INFINITY ? INFINITY : lse * kLog2e;
}

// Query tiles [lo, hi) of height BQ whose rows see some key in [ka, kb] of a
// sequence of M rows.
template <int MASK>
__device__ __forceinline__ void query_tiles(const BwdParams& p, int ka, int kb, int M, int BQ, int& lo, int& hi) {
    lo = hi = 0;
    if (ka > kb || M <= 0) return;
    const int i_lo = query_lo<MASK>(p.wr, ka), i_hi = query_hi<MASK>(p.wl, kb, M);
    if (i_lo > i_hi) return;
    lo = i_lo / BQ;
    hi = i_hi / BQ + 1;
}
// Do query rows r0 .. r0 + 31 and keys k0 .. k0 + 31 see each other at all
// (live), and does every row see every key (full; keys past N do not matter
// to the dK/dV kernels, which never store them).
template <int MASK>
__device__ __forceinline__ bool block_live(const BwdParams& p, int r0, int k0, int M, int N) {
    if (r0 >= M || k0 >= N) return false;
    return r0 <= query_hi<MASK>(p.wl, min(k0 + 31, N - 1), M) && r0 + 31 >= query_lo<MASK>(p.wr, k0);
}
template <int MASK>
__device__ __forceinline__ bool block_full(const BwdParams& p, int r0, int k0) {
    return key_lo<MASK>(p.wl, r0 + 31) <= k0 && key_hi<MASK>(p.wr, r0, INT_MAX) >= k0 + 31;
}
// Mask the S accumulator of rows rb + acc_row(r, h) (rb = the block's first
// row) against this lane's key.
template <int MASK>
__device__ __forceinline__ void mask_rows(const BwdParams& p, floatx16& sacc, int rb, int h, int key) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int q = rb + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key > key_hi<MASK>(p.wr, q, INT_MAX) || key < key_lo<MASK>(p.wl, q)) sacc[r] = -INFINITY;
    }
}

// 16-byte chunk XOR of LDS row r for tiles that are read both row-wise (A
// operand, 32 rows at one chunk: a quarter-wave covers 16 rows) and
// transposed (ds_read_b64_tr_b16: a half-wave covers 4 rows x 64 bytes).
// D = 128 (rows of 256 bytes, one full bank sweep): the low two bits of r
// pick the 64-byte quarter and bits 2..3 the chunk inside it, so 16
// consecutive rows hit 16 distinct chunk positions and 4 consecutive rows
// 4 distinct quarters.  D = 64 (128-byte rows, two per bank sweep): the same
// with bit 1 in place of bits 0..1 for the half of the row.
template <int D>
__device__ __forceinline__ int swz_rt(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Per-lane LDS offsets of the two fragment read patterns of a swizzled tile.
template <int D>
struct TileReads {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kDS = D / 16;
    static constexpr int kDB = D / 32;
    int row_off[kDS];    // A operand, rows of the 32-row block: lane = row, chunk 2 s + h
    int tr_lo[kDB];      // A operand of a transposed product, 16-row step: rows 0..7 of the step
    int tr_hi[kDB];      //   ... rows 8..15
    __device__ __forceinline__ void init(int lane) {
        const int l32 = lane & 31, h = lane >> 5;
#pragma unroll
        for (int s = 0; s < kDS; ++s) row_off[s] = l32 * kRowBytes + 16 * ((2 * s + h) ^ swz_rt<D>(l32));
        // ds_read_b64_tr_b16: lane 16 g + 4 t + a addresses row 4 (g >> 1) + t
        // (+ 8 for the high half) at d = 32 db + 16 (g & 1) + 4 a, and receives
        // the column d = 32 db + lane % 32 of the four rows its 16-lane group
        // addressed: slot t of the fragment is row 8 (t >> 2) + 4 (g >> 1) + t % 4
        // of the step, the order in which a 32x32 accumulator holds rows.
        const int g = lane >> 4, t = (lane >> 2) & 3, a = lane & 3;
        const int r_lo = 4 * (g >> 1) + t, r_hi = r_lo + 8;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
            const int c = 4 * db + 2 * (g & 1) + (a >> 1);
            tr_lo[db] = r_lo * kRowBytes + 16 * (c ^ swz_rt<D>(r_lo)) + 8 * (a & 1);
            tr_hi[db] = r_hi * kRowBytes + 16 * (c ^ swz_rt<D>(r_hi)) + 8 * (a & 1);
        }
    }
    // A operand of a product over d: rows 32 b .. 32 b + 31, d-step s
    template <typename V8>
    __device__ __forceinline__ V8 row(const char* tile, int b, int s) const {
        return *reinterpret_cast<const V8*>(tile + 32 * b * kRowBytes + row_off[s]);
    }
    // A operand of a product over the tile's rows: d block db, rows 16 step ..
    template <typename V8>
    __device__ __forceinline__ V8 tr(const char* tile, int step, int db) const {
        const char* p = tile + 16 * step * kRowBytes;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + tr_lo[db]));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + tr_hi[db]));
        return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// Byte offsets (inside a tile) of this lane's global -> LDS copies: wave w
// moves slots [w L 64, (w + 1) L 64); slot s is row s / CPR, physical chunk
// s % CPR, i.e. logical chunk (s % CPR) ^ swz_rt(row).
template <int D, int kLoads>
__device__ __forceinline__ void copy_offsets(uint32_t* off, int wave, int lane) {
    constexpr int kCPR = D / 8;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int slot = (wave * kLoads + i) * 64 + lane;
        const int r = slot / kCPR, c = slot % kCPR;
        off[i] = (uint32_t)(r * 2 * D + 16 * (c ^ swz_rt<D>(r)));
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (key tile, K/V head)
// ---------------------------------------------------------------------------
// D: head dim; BQ: query rows per streamed tile (32 or 64); NW: waves, each
// owning 32 consecutive keys.
template <int D, int BQ, int NW>
struct BwdKVTraits {
    static constexpr int kThreads = NW * 64;
    static constexpr int kBN = 32 * NW;      // keys per workgroup
    static constexpr int kQB = BQ / 32;      // 32-query blocks per tile
    static constexpr int kDB = D / 32;
    static constexpr int kDS = D / 16;
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kTileBytes = BQ * kRowBytes;
    static constexpr int kLoadsPerWave = BQ * (D / 8) / (64 * NW);
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BQ == 32 || BQ == 64, "query tile");
    static_assert(NW >= 2, "waves 0 and 1 stage L and Delta");
    static_assert(BQ * (D / 8) % (64 * NW) == 0, "loader split");
};

template <typename E, int D, int BQ, int NW, int WAVES_PER_SIMD, int MASK>
__global__ void __launch_bounds__(NW * 64, WAVES_PER_SIMD)
fa2_bwd_dkdv_kernel(const BwdParams p) {
    using T = BwdKVTraits<D, BQ, NW>;
    using V8 = typename Half<E>::v8;
    const E* __restrict__ Q = static_cast<const E*>(p.q);
    const E* __restrict__ K = static_cast<const E*>(p.k);
    const E* __restrict__ V = static_cast<const E*>(p.v);
    const E* __restrict__ dO = static_cast<const E*>(p.dout);
    E* __restrict__ dK = static_cast<E*>(p.dk);
    E* __restrict__ dV = static_cast<E*>(p.dv);
    const float c_log2 = p.c_log2;
    // double-buffered Q and dO tiles, and the tile's L (log2 units) and Delta
    __shared__ __attribute__((aligned(1024))) char sQ0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sO0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sQ1[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sO1[T::kTileBytes];
    __shared__ __attribute__((aligned(16))) float sL0[BQ], sL1[BQ], sD0[BQ], sD1[BQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // key tiles major (under a causal mask the first key tile has the most
    // query tiles), K/V heads fastest
    const int bkv = blockIdx.x % p.BHk;
    const int kt = blockIdx.x / p.BHk;
    const BwdSeq sq = bwd_seq(p, p.cu_q ? bkv / p.Hk : 0);
    const int M = sq.M, N = sq.N;
    const int kbase = kt * T::kBN;
    const int k0 = kbase + 32 * wave;  // first key of this wave
    const int key = k0 + l32;          // this lane's key

    // K and V rows of the wave's keys: B operands of S = Q K^T and dP = dO V^T
    const int64_t kvr = kv_row0(p, sq, bkv);
    const E* Kh = K + kvr * D;
    const E* Vh = V + kvr * D;
    V8 kf[T::kDS], vf[T::kDS];
#pragma unroll
    for (int s = 0; s < T::kDS; ++s) {
        if (key < N) {
            kf[s] = *reinterpret_cast<const V8*>(Kh + (int64_t)key * D + 16 * s + 8 * h);
            vf[s] = *reinterpret_cast<const V8*>(Vh + (int64_t)key * D + 16 * s + 8 * h);
        } else {
            kf[s] = V8{};
            vf[s] = V8{};
        }
    }

    // query tiles: every query head of the group, the tiles whose rows see
    // some key of the workgroup
    int qt0, qt1;
    query_tiles<MASK>(p, kbase, min(kbase + T::kBN, N) - 1, M, BQ, qt0, qt1);
    const int per_g = qt1 - qt0;
    const int n_it = p.G * per_g;

    floatx16 dkacc[T::kDB], dvacc[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) dkacc[db] = dvacc[db] = floatx16{};

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t cp_off[T::kLoadsPerWave];
    copy_offsets<D, T::kLoadsPerWave>(cp_off, wave, lane);
    TileReads<D> rd;
    rd.init(lane);

    auto tile_head = [&](int it, int& bh, int& qt) {
        const int g = it / per_g;
        qt = qt0 + (it - g * per_g);
        bh = bkv * p.G + g;
    };
    auto issue_tile = [&](int it, char* qdst, char* odst) {
        int bh, qt;
        tile_head(it, bh, qt);
        const int64_t qr = q_row0(p, sq, bh);
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BQ>(Q + qr * D, cp_off, wave_u, qt, M, qdst);
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BQ>(dO + qr * D, cp_off, wave_u, qt, M, odst);
    };
    // wave 0 fetches the tile's L (log2 units, l2_of), wave 1 its Delta
    // (0 past M)
    auto fetch_ld = [&](int it) -> float {
        int bh, qt;
        tile_head(it, bh, qt);
        const int row = qt * BQ + lane;
        if (lane >= BQ || wave > 1) return 0.f;
        const int64_t qr = q_row0(p, sq, bh);
        if (wave == 0) return l2_of(row < M ? p.lse[qr + row] : INFINITY);
        return row < M ? p.delta[qr + row] : 0.f;
    };
    auto store_ld = [&](float x, float* sl, float* sd) {
        if (lane < BQ) {
            if (wave == 0) sl[lane] = x;
            else if (wave == 1) sd[lane] = x;
        }
    };

    auto compute_tile = [&](int it, const char* qs, const char* os, const float* ls, const float* dls) {
        int bh, qt;
        tile_head(it, bh, qt);
        const int row0 = qt * BQ;
        // nothing to do unless some row of the tile sees some key of the wave
        bool live = false;
#pragma unroll
        for (int qb = 0; qb < T::kQB; ++qb) live = live || block_live<MASK>(p, row0 + 32 * qb, k0, M, N);
        if (!live) return;
        // S = Q K^T and dP = dO V^T (rows: queries, columns: the wave's keys)
        floatx16 sacc[T::kQB], pacc[T::kQB];
#pragma unroll
        for (int qb = 0; qb < T::kQB; ++qb) sacc[qb] = pacc[qb] = floatx16{};
#pragma unroll
        for (int s = 0; s < T::kDS; ++s) {
            V8 qa[T::kQB], oa[T::kQB];
#pragma unroll
            for (int qb = 0; qb < T::kQB; ++qb) {
                qa[qb] = rd.template row<V8>(qs, qb, s);
                oa[qb] = rd.template row<V8>(os, qb, s);
            }
#pragma unroll
            for (int qb = 0; qb < T::kQB; ++qb) {
                sacc[qb] = Half<E>::mfma(qa[qb], kf[s], sacc[qb]);
                pacc[qb] = Half<E>::mfma(oa[qb], vf[s], pacc[qb]);
            }
        }
        // P = exp2(S c - L2) and dS = P (dP - Delta), rounded once to 16 bits
        // as B operands of the dV and dK products; register r of the
        // accumulator holds query row0 + 32 qb + acc_row(r, h).
        bool full = true;  // every row of the tile sees every key of the wave
#pragma unroll
        for (int qb = 0; qb < T::kQB; ++qb) full = full && block_full<MASK>(p, row0 + 32 * qb, k0);
        uint32_t pw[T::kQB][2][4], sw[T::kQB][2][4];
#pragma unroll
        for (int qb = 0; qb < T::kQB; ++qb) {
            floatx4 l4[4], d4[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                l4[g] = *reinterpret_cast<const floatx4*>(ls + 32 * qb + 8 * g + 4 * h);
                d4[g] = *reinterpret_cast<const floatx4*>(dls + 32 * qb + 8 * g + 4 * h);
            }
            if (MASK != kMaskNone && !full) {
                __asm__ volatile("");  // keep this a branch, not a select per element
                mask_rows<MASK>(p, sacc[qb], row0 + 32 * qb, h, key);
            }
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(sacc[qb][r], c_log2, -l4[r >> 2][r & 3]));
                const float p1 = fast_exp2(fmaf(sacc[qb][r + 1], c_log2, -l4[r >> 2][(r & 3) + 1]));
                const float s0 = p0 * (pacc[qb][r] - d4[r >> 2][r & 3]);
                const float s1 = p1 * (pacc[qb][r + 1] - d4[r >> 2][(r & 3) + 1]);
                pw[qb][r >> 3][(r & 7) >> 1] = pack2<E>(p0, p1);
                sw[qb][r >> 3][(r & 7) >> 1] = pack2<E>(s0, s1);
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the tile's queries
#pragma unroll
        for (int qb = 0; qb < T::kQB; ++qb)
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                const V8 pb = __builtin_bit_cast(V8, u32x4{pw[qb][ms][0], pw[qb][ms][1], pw[qb][ms][2], pw[qb][ms][3]});
                const V8 sb = __builtin_bit_cast(V8, u32x4{sw[qb][ms][0], sw[qb][ms][1], sw[qb][ms][2], sw[qb][ms][3]});
                V8 oa[T::kDB], qa[T::kDB];
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) {
                    oa[db] = rd.template tr<V8>(os, 2 * qb + ms, db);
                    qa[db] = rd.template tr<V8>(qs, 2 * qb + ms, db);
                }
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) {
                    dvacc[db] = Half<E>::mfma(oa[db], pb, dvacc[db]);
                    dkacc[db] = Half<E>::mfma(qa[db], sb, dkacc[db]);
                }
            }
    };

    // ---- main loop, unrolled by two over the buffer pair
    if (n_it > 0) {
        issue_tile(0, sQ0, sO0);
        store_ld(fetch_ld(0), sL0, sD0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int it = 0; it < n_it; it += 2) {
        float nx = 0.f;
        if (it + 1 < n_it) {
            issue_tile(it + 1, sQ1, sO1);
            nx = fetch_ld(it + 1);
        }
        compute_tile(it, sQ0, sO0, sL0, sD0);
        if (it + 1 < n_it) store_ld(nx, sL1, sD1);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next tile have landed
        __syncthreads();
        if (it + 1 >= n_it) break;
        if (it + 2 < n_it) {
            issue_tile(it + 2, sQ0, sO0);
            nx = fetch_ld(it + 2);
        }
        compute_tile(it + 1, sQ1, sO1, sL1, sD1);
        if (it + 2 < n_it) store_ld(nx, sL0, sD0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: dK = scale dS^T Q, dV = P^T dO, rounded to nearest even
    if (key < N) {
        const float scale = p.scale;
        E* krow = dK + (kvr + key) * D;
        E* vrow = dV + (kvr + key) * D;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * db + 8 * g + 4 * h;
                const uint32_t k0w = pack2<E>(dkacc[db][4 * g + 0] * scale, dkacc[db][4 * g + 1] * scale);
                const uint32_t k1w = pack2<E>(dkacc[db][4 * g + 2] * scale, dkacc[db][4 * g + 3] * scale);
                *reinterpret_cast<uint2*>(krow + d) = make_uint2(k0w, k1w);
                const uint32_t v0w = pack2<E>(dvacc[db][4 * g + 0], dvacc[db][4 * g + 1]);
                const uint32_t v1w = pack2<E>(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]);
                *reinterpret_cast<uint2*>(vrow + d) = make_uint2(v0w, v1w);
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV with wave pairs: one workgroup of 8 waves per (128-key tile, K/V head)
// ---------------------------------------------------------------------------
// At D = 128 a wave that keeps its keys' K and V in VGPRs next to the dK and
// dV accumulators (192 VGPRs) leaves no room for a second wave on its SIMD,
// and a lone wave cannot overlap its own MFMA and VALU work.  Here the
// workgroup's K and V stay in LDS instead (read as B operands each tile), and
// waves w and w + 4 -- which share a SIMD -- own the same 32 keys and split
// each 64-row query tile: wave w takes rows 0..31, wave w + 4 rows 32..63.
// Each holds partial dK, dV of its keys; the pair's partials are summed
// through LDS once at the end.  Two waves per SIMD let one wave's MFMAs run
// while the other waits on LDS or works through its softmax-gradient VALU
// block.
template <int D>
struct BwdPairTraits {
    static constexpr int kNW = 8;
    static constexpr int kThreads = kNW * 64;
    static constexpr int kBN = 128;            // keys per workgroup
    static constexpr int kBQ = 64;             // query rows per streamed tile
    static constexpr int kDB = D / 32;
    static constexpr int kDS = D / 16;
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kQTileBytes = kBQ * kRowBytes;
    static constexpr int kKTileBytes = kBN * kRowBytes;
    static constexpr int kQLoads = kBQ * (D / 8) / (64 * kNW);
    static constexpr int kKLoads = kBN * (D / 8) / (64 * kNW);
    static constexpr int kPartBytes = 64 * kDB * 16 * 4;  // one wave's fp32 accumulator set
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(kQLoads >= 1 && kKLoads >= 1, "loader split");
    // the pair sum puts dK partials over the four Q/dO buffers and dV
    // partials over the K/V tiles
    static_assert(kPartBytes <= kQTileBytes && 2 * kPartBytes <= kKTileBytes, "pair sum space");
};

template <typename E, int D, int MASK>
__global__ void __launch_bounds__(512, 2)
fa2_bwd_dkdv_pair_kernel(const BwdParams p) {
    using T = BwdPairTraits<D>;
    using V8 = typename Half<E>::v8;
    const E* __restrict__ Q = static_cast<const E*>(p.q);
    const E* __restrict__ K = static_cast<const E*>(p.k);
    const E* __restrict__ V = static_cast<const E*>(p.v);
    const E* __restrict__ dO = static_cast<const E*>(p.dout);
    E* __restrict__ dK = static_cast<E*>(p.dk);
    E* __restrict__ dV = static_cast<E*>(p.dv);
    const float c_log2 = p.c_log2;
    // The Q/dO buffers are read twice per row block (as rows and transposed)
    // and carry the larger alignment, which places them first, below 64 KiB,
    // where their bases fit the DS instructions' 16-bit offset field; K and V
    // share one array so that V is K plus a constant offset.
    __shared__ __attribute__((aligned(T::kQTileBytes))) char sQ0[T::kQTileBytes];
    __shared__ __attribute__((aligned(T::kQTileBytes))) char sO0[T::kQTileBytes];
    __shared__ __attribute__((aligned(T::kQTileBytes))) char sQ1[T::kQTileBytes];
    __shared__ __attribute__((aligned(T::kQTileBytes))) char sO1[T::kQTileBytes];
    __shared__ __attribute__((aligned(1024))) char sKV[2 * T::kKTileBytes];
    char* const sK = sKV;
    char* const sV = sKV + T::kKTileBytes;
    __shared__ __attribute__((aligned(16))) float sL0[T::kBQ], sL1[T::kBQ], sD0[T::kBQ], sD1[T::kBQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kb = wave & 3;   // the wave's 32-key block of the workgroup's keys
    const int qb = wave >> 2;  // the wave's 32-row block of each query tile
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // key tiles major (under a causal mask the first key tile has the most
    // query tiles), K/V heads fastest
    const int bkv = blockIdx.x % p.BHk;
    const int kt = blockIdx.x / p.BHk;
    const BwdSeq sq = bwd_seq(p, p.cu_q ? bkv / p.Hk : 0);
    const int M = sq.M, N = sq.N;
    const int64_t kvr = kv_row0(p, sq, bkv);
    const int kbase = kt * T::kBN;
    const int k0 = kbase + 32 * kb;  // first key of this wave
    const int key = k0 + l32;        // this lane's key

    // query tiles: every query head of the group, the tiles whose rows see
    // some key of the workgroup
    int qt0, qt1;
    query_tiles<MASK>(p, kbase, min(kbase + T::kBN, N) - 1, M, T::kBQ, qt0, qt1);
    const int per_g = qt1 - qt0;
    const int n_it = p.G * per_g;

    floatx16 dkacc[T::kDB], dvacc[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) dkacc[db] = dvacc[db] = floatx16{};

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t q_off[T::kQLoads], k_off[T::kKLoads];
    copy_offsets<D, T::kQLoads>(q_off, wave, lane);
    copy_offsets<D, T::kKLoads>(k_off, wave, lane);
    TileReads<D> rd;
    rd.init(lane);
    // per-lane read offsets with the wave's row block folded in (the wave
    // index is uniform, but a value derived from the thread index is treated
    // as per-lane; folding it here keeps an add off every read)
    int q_row[T::kDS], k_row[T::kDS], q_tr_lo[T::kDB], q_tr_hi[T::kDB];
#pragma unroll
    for (int s = 0; s < T::kDS; ++s) {
        q_row[s] = 32 * qb * T::kRowBytes + rd.row_off[s];
        k_row[s] = 32 * kb * T::kRowBytes + rd.row_off[s];
    }
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) {
        q_tr_lo[db] = 32 * qb * T::kRowBytes + rd.tr_lo[db];
        q_tr_hi[db] = 32 * qb * T::kRowBytes + rd.tr_hi[db];
    }
    auto tr_read = [&](const char* tile, int ms, int db) {
        const char* p = tile + 16 * ms * T::kRowBytes;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + q_tr_lo[db]));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + q_tr_hi[db]));
        return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    auto tile_head = [&](int it, int& bh, int& qt) {
        const int g = it / per_g;
        qt = qt0 + (it - g * per_g);
        bh = bkv * p.G + g;
    };
    auto issue_tile = [&](int it, char* qdst, char* odst) {
        int bh, qt;
        tile_head(it, bh, qt);
        const int64_t qr = q_row0(p, sq, bh);
        copy_tile_to_lds<T::kQLoads, T::kRowBytes, T::kBQ>(Q + qr * D, q_off, wave_u, qt, M, qdst);
        copy_tile_to_lds<T::kQLoads, T::kRowBytes, T::kBQ>(dO + qr * D, q_off, wave_u, qt, M, odst);
    };
    // wave 0 fetches the tile's L (log2 units, l2_of), wave 1 its Delta
    // (0 past M)
    auto fetch_ld = [&](int it) -> float {
        int bh, qt;
        tile_head(it, bh, qt);
        const int row = qt * T::kBQ + lane;
        if (wave > 1) return 0.f;
        const int64_t qr = q_row0(p, sq, bh);
        if (wave == 0) return l2_of(row < M ? p.lse[qr + row] : INFINITY);
        return row < M ? p.delta[qr + row] : 0.f;
    };
    auto store_ld = [&](float x, float* sl, float* sd) {
        if (wave == 0) sl[lane] = x;
        else if (wave == 1) sd[lane] = x;
    };

    auto compute_tile = [&](int it, const char* qs, const char* os, const float* ls, const float* dls) {
        int bh, qt;
        tile_head(it, bh, qt);
        const int r0 = qt * T::kBQ + 32 * qb;  // first query row of the wave's block
        // nothing to do unless some row of the block sees some key of the wave
        if (!block_live<MASK>(p, r0, k0, M, N)) return;
        // S = Q K^T and dP = dO V^T (rows: the block's queries, columns: the
        // wave's keys), K and V rows read from LDS as B operands
        floatx16 sacc = floatx16{}, pacc = floatx16{};
#pragma unroll
        for (int s = 0; s < T::kDS; ++s) {
            const V8 qa = *reinterpret_cast<const V8*>(qs + q_row[s]);
            const V8 oa = *reinterpret_cast<const V8*>(os + q_row[s]);
            const V8 kf = *reinterpret_cast<const V8*>(sK + k_row[s]);
            const V8 vf = *reinterpret_cast<const V8*>(sV + k_row[s]);
            sacc = Half<E>::mfma(qa, kf, sacc);
            pacc = Half<E>::mfma(oa, vf, pacc);
        }
        // P = exp2(S c - L2), dS = P (dP - Delta); register r holds query
        // r0 + acc_row(r, h)
        if (MASK != kMaskNone && !block_full<MASK>(p, r0, k0)) {
            __asm__ volatile("");  // keep this a branch, not a select per element
            mask_rows<MASK>(p, sacc, r0, h, key);
        }
        uint32_t pw[2][4], sw[2][4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const floatx4 l4 = *reinterpret_cast<const floatx4*>(ls + 32 * qb + 8 * g + 4 * h);
            const floatx4 d4 = *reinterpret_cast<const floatx4*>(dls + 32 * qb + 8 * g + 4 * h);
#pragma unroll
            for (int u = 0; u < 4; u += 2) {
                const int r = 4 * g + u;
                const float p0 = fast_exp2(fmaf(sacc[r], c_log2, -l4[u]));
                const float p1 = fast_exp2(fmaf(sacc[r + 1], c_log2, -l4[u + 1]));
                pw[r >> 3][(r & 7) >> 1] = pack2<E>(p0, p1);
                sw[r >> 3][(r & 7) >> 1] = pack2<E>(p0 * (pacc[r] - d4[u]), p1 * (pacc[r + 1] - d4[u + 1]));
            }
        }
        // dV^T += dO^T P, dK^T += Q^T dS over the block's 32 rows
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
            const V8 pb = __builtin_bit_cast(V8, u32x4{pw[ms][0], pw[ms][1], pw[ms][2], pw[ms][3]});
            const V8 sb = __builtin_bit_cast(V8, u32x4{sw[ms][0], sw[ms][1], sw[ms][2], sw[ms][3]});
#pragma unroll
            for (int db = 0; db < T::kDB; ++db) {
                const V8 oa = tr_read(os, ms, db);
                const V8 qa = tr_read(qs, ms, db);
                dvacc[db] = Half<E>::mfma(oa, pb, dvacc[db]);
                dkacc[db] = Half<E>::mfma(qa, sb, dkacc[db]);
            }
        }
    };

    // ---- prologue: the workgroup's K and V tiles, the first Q/dO tile
    if (n_it > 0) {
        copy_tile_to_lds<T::kKLoads, T::kRowBytes, T::kBN>(K + kvr * D, k_off, wave_u, kt, N, sK);
        copy_tile_to_lds<T::kKLoads, T::kRowBytes, T::kBN>(V + kvr * D, k_off, wave_u, kt, N, sV);
        issue_tile(0, sQ0, sO0);
        store_ld(fetch_ld(0), sL0, sD0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // ---- main loop, unrolled by two over the Q/dO buffer pair
    for (int it = 0; it < n_it; it += 2) {
        float nx = 0.f;
        if (it + 1 < n_it) {
            issue_tile(it + 1, sQ1, sO1);
            nx = fetch_ld(it + 1);
        }
        compute_tile(it, sQ0, sO0, sL0, sD0);
        if (it + 1 < n_it) store_ld(nx, sL1, sD1);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next tile have landed
        __syncthreads();
        if (it + 1 >= n_it) break;
        if (it + 2 < n_it) {
            issue_tile(it + 2, sQ0, sO0);
            nx = fetch_ld(it + 2);
        }
        compute_tile(it + 1, sQ1, sO1, sL1, sD1);
        if (it + 2 < n_it) store_ld(nx, sL0, sD0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- pair sum through LDS: waves 4..7 hand their partials to waves 0..3
    // (dK partials over the Q/dO buffers, dV partials over the K/V tiles; the
    // loop's last barrier has retired every read of them)
    char* const kpart = kb == 0 ? sQ0 : kb == 1 ? sO0 : kb == 2 ? sQ1 : sO1;
    char* const vpart = (kb < 2 ? sK : sV) + (kb & 1) * T::kPartBytes;
    if (qb == 1) {
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int off = ((db * 4 + g) * 64 + lane) * 16;
                *reinterpret_cast<floatx4*>(kpart + off) =
                    floatx4{dkacc[db][4 * g], dkacc[db][4 * g + 1], dkacc[db][4 * g + 2], dkacc[db][4 * g + 3]};
                *reinterpret_cast<floatx4*>(vpart + off) =
                    floatx4{dvacc[db][4 * g], dvacc[db][4 * g + 1], dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]};
            }
    }
    __syncthreads();
    // ---- epilogue (waves 0..3): dK = scale dS^T Q, dV = P^T dO, rounded to
    // nearest even
    if (qb == 0 && key < N) {
        const float scale = p.scale;
        E* krow = dK + (kvr + key) * D;
        E* vrow = dV + (kvr + key) * D;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int off = ((db * 4 + g) * 64 + lane) * 16;
                const floatx4 pk = *reinterpret_cast<const floatx4*>(kpart + off);
                const floatx4 pv = *reinterpret_cast<const floatx4*>(vpart + off);
                const int d = 32 * db + 8 * g + 4 * h;
                const uint32_t k0w = pack2<E>((dkacc[db][4 * g + 0] + pk[0]) * scale, (dkacc[db][4 * g + 1] + pk[1]) * scale);
                const uint32_t k1w = pack2<E>((dkacc[db][4 * g + 2] + pk[2]) * scale, (dkacc[db][4 * g + 3] + pk[3]) * scale);
                *reinterpret_cast<uint2*>(krow + d) = make_uint2(k0w, k1w);
                const uint32_t v0w = pack2<E>(dvacc[db][4 * g + 0] + pv[0], dvacc[db][4 * g + 1] + pv[1]);
                const uint32_t v1w = pack2<E>(dvacc[db][4 * g + 2] + pv[2], dvacc[db][4 * g + 3] + pv[3]);
                *reinterpret_cast<uint2*>(vrow + d) = make_uint2(v0w, v1w);
            }
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (query tile, query head)
// ---------------------------------------------------------------------------
// D: head dim; BN: keys per streamed K/V tile (multiple of 32); NW: waves,
// each owning 32 consecutive query rows.
template <int D, int BN, int NW>
struct BwdQTraits {
    static constexpr int kThreads = NW * 64;
    static constexpr int kBM = 32 * NW;      // query rows per workgroup
    static constexpr int kKB = BN / 32;
    static constexpr int kDB = D / 32;
    static constexpr int kDS = D / 16;
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kTileBytes = BN * kRowBytes;
    static constexpr int kLoadsPerWave = BN * (D / 8) / (64 * NW);
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BN % 32 == 0, "key tile");
    static_assert(BN * (D / 8) % (64 * NW) == 0, "loader split");
};

template <typename E, int D, int BN, int NW, int WAVES_PER_SIMD, int MASK>
__global__ void __launch_bounds__(NW * 64, WAVES_PER_SIMD)
fa2_bwd_dq_kernel(const BwdParams p) {
    using T = BwdQTraits<D, BN, NW>;
    using V8 = typename Half<E>::v8;
    const E* __restrict__ Q = static_cast<const E*>(p.q);
    const E* __restrict__ K = static_cast<const E*>(p.k);
    const E* __restrict__ V = static_cast<const E*>(p.v);
    const E* __restrict__ dO = static_cast<const E*>(p.dout);
    E* __restrict__ dQ = static_cast<E*>(p.dq);
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

    // query tiles major (heaviest first under a causal mask), heads fastest
    const int bh = blockIdx.x % p.BH;
    int qt = blockIdx.x / p.BH;
    if (MASK == kMaskCausal) qt = p.n_qt - 1 - qt;
    const int bkv = p.G == 1 ? bh : bh / p.G;
    const BwdSeq sq = bwd_seq(p, p.cu_q ? bh / p.H : 0);
    const int M = sq.M, N = sq.N;
    const int64_t qr = q_row0(p, sq, bh), kvr = kv_row0(p, sq, bkv);
    const int qw0 = qt * T::kBM + 32 * wave;  // first query row of this wave
    const int qw1 = min(qw0 + 32, M) - 1;     // its last row
    const int query = qw0 + l32;              // this lane's query row

    // Q and dO rows of the lane's query: B operands of S^T = K Q^T and
    // dP^T = V dO^T; L (log2 units) and Delta of the row
    const E* Qh = Q + qr * D;
    const E* dOh = dO + qr * D;
    V8 qf[T::kDS], of[T::kDS];
#pragma unroll
    for (int s = 0; s < T::kDS; ++s) {
        if (query < M) {
            qf[s] = *reinterpret_cast<const V8*>(Qh + (int64_t)query * D + 16 * s + 8 * h);
            of[s] = *reinterpret_cast<const V8*>(dOh + (int64_t)query * D + 16 * s + 8 * h);
        } else {
            qf[s] = V8{};
            of[s] = V8{};
        }
    }
    const float l2 = l2_of(query < M ? p.lse[qr + query] : INFINITY);
    // Delta = rowsum(dO o O) of the row (fp32 sums of the 16-bit products):
    // each lane half holds half of the row's dO; the matching O values are
    // read once, and the two halves' sums are exchanged.  Stored for the
    // dK/dV kernel (0 past M, not stored).
    float dl;
    {
        using V2 = typename Half<E>::v2;
        const E* Oh = static_cast<const E*>(p.o) + qr * D;
        float part = 0.f;
        if (query < M) {
#pragma unroll
            for (int s = 0; s < T::kDS; ++s) {
                const V8 ov = *reinterpret_cast<const V8*>(Oh + (int64_t)query * D + 16 * s + 8 * h);
#pragma unroll
                for (int j = 0; j < 8; j += 2)
                    part = Half<E>::dot2(V2{of[s][j], of[s][j + 1]}, V2{ov[j], ov[j + 1]}, part);
            }
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        dl = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if (h == 0 && query < M) p.delta[qr + query] = dl;
    }

    // K/V tiles [t0, t0 + n_kv): from the first key the workgroup's first row
    // sees to the last key its last row sees; the wave needs [w0, w1) of them
    int t0 = 0, n_kv = 0, w0 = 0, w1 = 0;
    {
        const int r0 = qt * T::kBM, r1 = min(r0 + T::kBM, M) - 1;
        if (r0 <= r1) {
            const int klo = key_lo<MASK>(p.wl, r0), khi = key_hi<MASK>(p.wr, r1, N);
            if (klo <= khi) {
                t0 = klo / BN;
                n_kv = khi / BN + 1 - t0;
            }
        }
        if (qw0 <= qw1) {
            const int klo = key_lo<MASK>(p.wl, qw0), khi = key_hi<MASK>(p.wr, qw1, N);
            if (klo <= khi) {
                w0 = klo / BN - t0;
                w1 = khi / BN + 1 - t0;
            }
        }
    }

    floatx16 dqacc[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) dqacc[db] = floatx16{};

    const E* Kh = K + kvr * D;
    const E* Vh = V + kvr * D;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t cp_off[T::kLoadsPerWave];
    copy_offsets<D, T::kLoadsPerWave>(cp_off, wave, lane);
    TileReads<D> rd;
    rd.init(lane);
    // kt: local tile, K/V tile t0 + kt of the sequence
    auto issue_tile = [&](int kt, char* kdst, char* vdst) {
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BN>(Kh, cp_off, wave_u, t0 + kt, N, kdst);
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BN>(Vh, cp_off, wave_u, t0 + kt, N, vdst);
    };

    auto compute_tile = [&](int kt, const char* ks, const char* vs) {
        if (kt < w0 || kt >= w1) return;
        // S^T = K Q^T, dP^T = V dO^T (rows: keys, columns: the wave's queries)
        floatx16 sacc[T::kKB], pacc[T::kKB];
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb) sacc[kb] = pacc[kb] = floatx16{};
        // K and V operands read from LDS two steps ahead of their MFMAs (the
        // scheduling fences keep the reads from sinking next to their uses)
        constexpr int kSteps = T::kDS * T::kKB;
        constexpr int kAhead = 2;
        V8 kr[kAhead + 1], vr[kAhead + 1];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
            kr[i] = rd.template row<V8>(ks, i % T::kKB, i / T::kKB);
            vr[i] = rd.template row<V8>(vs, i % T::kKB, i / T::kKB);
        }
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            if (i + kAhead < kSteps) {
                const int j = i + kAhead;
                kr[j % (kAhead + 1)] = rd.template row<V8>(ks, j % T::kKB, j / T::kKB);
                vr[j % (kAhead + 1)] = rd.template row<V8>(vs, j % T::kKB, j / T::kKB);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int s = i / T::kKB, kb = i % T::kKB;
            sacc[kb] = Half<E>::mfma(kr[i % (kAhead + 1)], qf[s], sacc[kb]);
            pacc[kb] = Half<E>::mfma(vr[i % (kAhead + 1)], of[s], pacc[kb]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the A operands of dQ^T += K^T dS^T, read now so that their latency
        // passes during the softmax-gradient work below
        V8 kt_a[T::kKB][2][T::kDB];
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) kt_a[kb][ms][db] = rd.template tr<V8>(ks, 2 * kb + ms, db);
        __builtin_amdgcn_sched_barrier(0);
        // boundary tiles only: keys past N, or outside some row's causal or
        // window range; key kbase + 32 kb + acc_row(r, h) is visible iff its
        // compile-time part lies in [lim_lo, lim]
        const int kbase = (t0 + kt) * BN;
        if (kbase + BN > N || (MASK != kMaskNone && kbase + BN - 1 > key_hi<MASK>(p.wr, qw0, N)) ||
            (MASK == kMaskLocal && kbase < key_lo<MASK>(p.wl, qw1))) {
            __asm__ volatile("");
            const int lim = key_hi<MASK>(p.wr, query, N) - kbase - 4 * h;
            const int lim_lo = key_lo<MASK>(p.wl, query) - kbase - 4 * h;
#pragma unroll
            for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int idx = 32 * kb + 8 * (r >> 2) + (r & 3);
                    if (idx > lim || (MASK == kMaskLocal && idx < lim_lo)) sacc[kb][r] = -INFINITY;
                }
        }
        // dS^T = P^T (dP^T - Delta), rounded once: B operand of dQ^T += K^T dS^T
        uint32_t sw[T::kKB][2][4];
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(sacc[kb][r], c_log2, -l2));
                const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], c_log2, -l2));
                sw[kb][r >> 3][(r & 7) >> 1] = pack2<E>(p0 * (pacc[kb][r] - dl), p1 * (pacc[kb][r + 1] - dl));
            }
#pragma unroll
        for (int kb = 0; kb < T::kKB; ++kb)
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                const V8 sb = __builtin_bit_cast(V8, u32x4{sw[kb][ms][0], sw[kb][ms][1], sw[kb][ms][2], sw[kb][ms][3]});
#pragma unroll
                for (int db = 0; db < T::kDB; ++db) dqacc[db] = Half<E>::mfma(kt_a[kb][ms][db], sb, dqacc[db]);
            }
    };

    // ---- main loop, unrolled by two over the buffer pair
    if (n_kv > 0) issue_tile(0, sK0, sV0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < n_kv; kt += 2) {
        if (kt + 1 < n_kv) issue_tile(kt + 1, sK1, sV1);
        compute_tile(kt, sK0, sV0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 >= n_kv) break;
        if (kt + 2 < n_kv) issue_tile(kt + 2, sK0, sV0);
        compute_tile(kt + 1, sK1, sV1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: dQ = scale dS K, rounded to nearest even
    if (query < M) {
        const float scale = p.scale;
        E* row = dQ + (qr + query) * D;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * db + 8 * g + 4 * h;
                const uint32_t w0 = pack2<E>(dqacc[db][4 * g + 0] * scale, dqacc[db][4 * g + 1] * scale);
                const uint32_t w1 = pack2<E>(dqacc[db][4 * g + 2] * scale, dqacc[db][4 * g + 3] * scale);
                *reinterpret_cast<uint2*>(row + d) = make_uint2(w0, w1);
            }
    }
}

// ---------------------------------------------------------------------------
// fp32 backward (v_mfma_f32_32x32x2_f32: true fp32 products, P and dS kept in
// fp32 as MFMA operands)
// ---------------------------------------------------------------------------
// MFMA step s of a product over d contracts d = h D/2 + s in lane half h of
// both operands (as in the fp32 forward), so a lane reads four consecutive
// d of a row at once (row-wise reads: 16 consecutive rows at one 16-byte
// chunk per quarter-wave); step r of a product over the rows of a 32-row
// block contracts rows acc_row(r, 0) and acc_row(r, 1), the rows whose P (or
// dS) the lane's accumulator register r holds (column reads: 32 floats of d
// of row r in lanes 0-31 and of row r + 4 in lanes 32-63).  Streamed tiles
// reach LDS by direct buffer-to-LDS copies into unpadded rows whose 16-byte
// chunks are XORed with swz_f32b(row): its low 4 bits spread the row-wise
// reads over 16 bank groups, and its bit 3 (row bit 3 ^ row bit 2) puts rows
// r and r + 4 in opposite halves of the bank space for the column reads.

// Delta = rowsum(dO o O): D / 4 lanes per row, 16 bytes each.
template <int D>
__global__ void __launch_bounds__(256)
fa2_bwd_delta_f32_kernel(const float* __restrict__ O, const float* __restrict__ dO, float* __restrict__ delta,
                         int rows) {
    constexpr int kLanes = D / 4;
    constexpr int kRowsPerWave = 64 / kLanes;
    const int lane = threadIdx.x & 63;
    const int row = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kRowsPerWave + lane / kLanes;
    const int c = lane % kLanes;
    float acc = 0.f;
    if (row < rows) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(O + (int64_t)row * D + 4 * c);
        const floatx4 b = *reinterpret_cast<const floatx4*>(dO + (int64_t)row * D + 4 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(a[i], b[i], acc);
    }
#pragma unroll
    for (int off = kLanes / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && c == 0) delta[row] = acc;
}

template <int D>
struct BwdF32Traits {
    static constexpr int kNW = 4;
    static constexpr int kThreads = kNW * 64;
    static constexpr int kRows = 32;                  // rows per streamed tile (queries or keys)
    static constexpr int kBlock = 32 * kNW;           // keys (dK/dV) or queries (dQ) per workgroup
    static constexpr int kDB = D / 32;
    static constexpr int kHalfD = D / 2;
    static constexpr int kRowBytes = D * 4;
    static constexpr int kCPR = D / 4;                // 16-byte chunks per row
    static constexpr int kTileBytes = kRows * kRowBytes;
    static constexpr int kLoadsPerWave = kRows * kCPR / (64 * kNW);  // per tensor per tile
    // two waves per SIMD at D = 64; at D = 128 the wave's K, V (Q, dO) rows
    // and its two accumulators alone take 256 registers
    static constexpr int kWavesPerSimd = D == 64 ? 2 : 1;
    static_assert(D == 64 || D == 128, "head dim");
    static_assert((kRows * kCPR) % (64 * kNW) == 0, "loader split");
};

__device__ __forceinline__ int swz_f32b(int r) { return (r & 15) ^ (8 * ((r >> 2) & 1)); }

// This lane's byte offsets inside a streamed tile (row * row bytes +
// swizzled chunk): wave w moves chunks [w*L*64, (w+1)*L*64), LDS slot s holds
// row s / CPR, physical chunk s % CPR.
template <int D>
struct F32Stream {
    using T = BwdF32Traits<D>;
    uint32_t off[T::kLoadsPerWave];
    __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < T::kLoadsPerWave; ++i) {
            const int slot = (wave * T::kLoadsPerWave + i) * 64 + lane;
            const int r = slot / T::kCPR, c = slot % T::kCPR;
            off[i] = (uint32_t)(r * T::kRowBytes + 16 * (c ^ swz_f32b(r)));
        }
    }
};

// Row-wise operand: floats d = h D/2 + s .. + 3 of row l32 (s % 4 == 0); `lane_row`
// is l32 * row bytes, `lane_xor` the lane's part of the chunk index XOR.
template <int D>
__device__ __forceinline__ floatx4 f32_row_read(const char* tile, int lane_row, int lane_xor, int s) {
    return *reinterpret_cast<const floatx4*>(tile + lane_row + 16 * (lane_xor ^ (s / 4)));
}
// Column operand of step r, block db: d = 32 db + l32 of row acc_row(r, h);
// `col_lane[db]` holds the lane's part (row 4h, chunk and in-chunk offset).
template <int D>
__device__ __forceinline__ float f32_col_read(const char* tile, const int* col_lane, int r, int db) {
    constexpr int kRowBytes = D * 4;
    const int rbase = (8 * (r >> 2) + (r & 3)) * kRowBytes;
    const int kx = 16 * ((r & 3) | (8 * ((r >> 2) & 1)));
    return *reinterpret_cast<const float*>(tile + rbase + (col_lane[db] ^ kx));
}
// The lane parts of the two reads.  Row-wise: chunk (h D/8 + s/4) ^ swz(l32)
// = (h D/8 ^ swz(l32)) ^ s/4.  Column: row acc_row(r, h) = 8(r>>2) + 4h +
// (r&3), whose swz is ((r&3) | 8((r>>2)&1)) ^ 12h, so the chunk
// (8 db + l32/4) ^ swz splits into a lane part and a step constant.
// The XORs make every operand address a lane value combined with a step
// constant, which the compiler would hoist out of the tile loop into one
// register per address; passing the lane values through an empty asm at the
// top of each tile keeps them in a few registers and costs one VALU per read.
template <int N>
__device__ __forceinline__ void opaque_lanes(int& a, int* b) {
    __asm__ volatile("" : "+v"(a));
#pragma unroll
    for (int i = 0; i < N; ++i) __asm__ volatile("" : "+v"(b[i]));
}
template <int D>
__device__ __forceinline__ void f32_read_lanes(int l32, int h, int& lane_row, int& lane_xor, int* col_lane) {
    constexpr int kRowBytes = D * 4;
    lane_row = l32 * kRowBytes;
    lane_xor = (h * (D / 8)) ^ swz_f32b(l32);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
        col_lane[db] = 4 * h * kRowBytes + 16 * ((8 * db + (l32 >> 2)) ^ (12 * h)) + 4 * (l32 & 3);
}

// dK, dV: one workgroup of 4 waves per (128-key tile, K/V head); each wave
// owns 32 keys and keeps their K and V rows in registers; Q and dO stream
// through LDS 32 rows at a time.
template <int D, int MASK>
__global__ void __launch_bounds__(256, BwdF32Traits<D>::kWavesPerSimd)
fa2_bwd_dkdv_f32_kernel(const BwdParams p) {
    using T = BwdF32Traits<D>;
    const float* __restrict__ Q = static_cast<const float*>(p.q);
    const float* __restrict__ K = static_cast<const float*>(p.k);
    const float* __restrict__ V = static_cast<const float*>(p.v);
    const float* __restrict__ dO = static_cast<const float*>(p.dout);
    float* __restrict__ dK = static_cast<float*>(p.dk);
    float* __restrict__ dV = static_cast<float*>(p.dv);
    const float c_log2 = p.c_log2;
    __shared__ __attribute__((aligned(1024))) char sQ0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sO0[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sQ1[T::kTileBytes];
    __shared__ __attribute__((aligned(1024))) char sO1[T::kTileBytes];
    __shared__ __attribute__((aligned(16))) float sL0[T::kRows], sD0[T::kRows], sL1[T::kRows], sD1[T::kRows];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    // key tiles major (under a causal mask the first key tile has the most
    // query tiles), K/V heads fastest
    const int bkv = blockIdx.x % p.BHk;
    const int kt = blockIdx.x / p.BHk;
    const BwdSeq sq = bwd_seq(p, p.cu_q ? bkv / p.Hk : 0);
    const int M = sq.M, N = sq.N;
    const int64_t kvr = kv_row0(p, sq, bkv);
    const int kbase = kt * T::kBlock;
    const int k0 = kbase + 32 * wave;  // first key of this wave
    const int key = k0 + l32;          // this lane's key

    // K and V rows of the lane's key, d half h: B operands of S = Q K^T and
    // dP = dO V^T
    float kf[T::kHalfD], vf[T::kHalfD];
#pragma unroll
    for (int s = 0; s < T::kHalfD; s += 4) {
        floatx4 x = floatx4{0.f, 0.f, 0.f, 0.f}, y = x;
        if (key < N) {
            x = *reinterpret_cast<const floatx4*>(K + (kvr + key) * D + h * T::kHalfD + s);
            y = *reinterpret_cast<const floatx4*>(V + (kvr + key) * D + h * T::kHalfD + s);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            kf[s + u] = x[u];
            vf[s + u] = y[u];
        }
    }

    // query tiles: every query head of the group, the 32-row tiles whose rows
    // see some key of the workgroup
    int qt0, qt1;
    query_tiles<MASK>(p, kbase, min(kbase + T::kBlock, N) - 1, M, T::kRows, qt0, qt1);
    const int per_g = qt1 - qt0;
    const int n_it = p.G * per_g;

    floatx16 dkacc[T::kDB], dvacc[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) dkacc[db] = dvacc[db] = floatx16{};

    auto tile_head = [&](int it, int& bh, int& qt) {
        const int g = it / per_g;
        qt = qt0 + (it - g * per_g);
        bh = bkv * p.G + g;
    };
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    F32Stream<D> st;
    st.init(wave, lane);
    int lane_row, lane_xor, col_lane[T::kDB];
    f32_read_lanes<D>(l32, h, lane_row, lane_xor, col_lane);

    // Q and dO rows of query tile `it` into LDS (rows past M re-read row M-1;
    // their L is +inf, so P = dS = 0 there); wave 0 loads the tile's L (log2
    // units), wave 1 its Delta, into a register until the tile's buffer is free
    float ld_next = 0.f;
    auto issue = [&](int it, char* qdst, char* odst) __attribute__((always_inline)) {
        int bh, qt;
        tile_head(it, bh, qt);
        const int64_t qr = q_row0(p, sq, bh);
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, T::kRows>(Q + qr * D, st.off, wave_u, qt, M, qdst);
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, T::kRows>(dO + qr * D, st.off, wave_u, qt, M, odst);
        const int row = qt * T::kRows + lane;
        if (wave == 0) ld_next = l2_of(row < M ? p.lse[qr + row] : INFINITY);
        else if (wave == 1) ld_next = row < M ? p.delta[qr + row] : 0.f;
    };
    auto stash = [&](float* sl, float* sd) __attribute__((always_inline)) {
        if (lane < T::kRows) {
            if (wave == 0) sl[lane] = ld_next;
            else if (wave == 1) sd[lane] = ld_next;
        }
    };

    auto compute_tile = [&](int it, const char* qs, const char* os, const float* sl, const float* sd)
                            __attribute__((always_inline)) {
        int bh, qt;
        tile_head(it, bh, qt);
        const int r0 = qt * T::kRows;
        if (!block_live<MASK>(p, r0, k0, M, N)) return;
        int lx = lane_xor, cl[T::kDB];
#pragma unroll
        for (int db = 0; db < T::kDB; ++db) cl[db] = col_lane[db];
        opaque_lanes<T::kDB>(lx, cl);
        // S = Q K^T and dP = dO V^T (rows: the tile's queries, columns: the
        // wave's keys)
        floatx16 sacc = floatx16{}, pacc = floatx16{};
#pragma unroll
        for (int s = 0; s < T::kHalfD; s += 4) {
            const floatx4 qa = f32_row_read<D>(qs, lane_row, lx, s);
            const floatx4 oa = f32_row_read<D>(os, lane_row, lx, s);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[u], kf[s + u], sacc, 0, 0, 0);
                pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(oa[u], vf[s + u], pacc, 0, 0, 0);
            }
        }
        if (MASK != kMaskNone && !block_full<MASK>(p, r0, k0)) {
            __asm__ volatile("");  // keep this a branch, not a select per element
            mask_rows<MASK>(p, sacc, r0, h, key);
        }
        // P = exp2(S c - L2), dS = P (dP - Delta); register r holds query
        // r0 + acc_row(r, h)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const floatx4 l4 = *reinterpret_cast<const floatx4*>(&sl[8 * g + 4 * h]);
            const floatx4 d4 = *reinterpret_cast<const floatx4*>(&sd[8 * g + 4 * h]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float pv = fast_exp2(fmaf(sacc[4 * g + u], c_log2, -l4[u]));
                sacc[4 * g + u] = pv;
                pacc[4 * g + u] = pv * (pacc[4 * g + u] - d4[u]);
            }
        }
        // dV^T += dO^T P and dK^T += Q^T dS: step r contracts the rows whose
        // P and dS the lane's register r holds
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int db = 0; db < T::kDB; ++db) {
                dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(f32_col_read<D>(os, cl, r, db), sacc[r], dvacc[db], 0, 0, 0);
                dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(f32_col_read<D>(qs, cl, r, db), pacc[r], dkacc[db], 0, 0, 0);
            }
        }
    };

    // ---- main loop, unrolled by two over the buffer pair so that every LDS
    // access names its buffer (the copy in flight never aliases the one read)
    if (n_it > 0) {
        issue(0, sQ0, sO0);
        stash(sL0, sD0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int it = 0; it < n_it; it += 2) {
        if (it + 1 < n_it) issue(it + 1, sQ1, sO1);
        compute_tile(it, sQ0, sO0, sL0, sD0);
        if (it + 1 < n_it) stash(sL1, sD1);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next tile have landed
        __syncthreads();
        if (it + 1 >= n_it) break;
        if (it + 2 < n_it) issue(it + 2, sQ0, sO0);
        compute_tile(it + 1, sQ1, sO1, sL1, sD1);
        if (it + 2 < n_it) stash(sL0, sD0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: dK = scale dS^T Q, dV = P^T dO; register r of block db
    // holds d = 32 db + acc_row(r, h) of the lane's key
    if (key < N) {
        const float scale = p.scale;
        float* krow = dK + (kvr + key) * D;
        float* vrow = dV + (kvr + key) * D;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * db + 8 * g + 4 * h;
                *reinterpret_cast<floatx4*>(krow + d) =
                    floatx4{dkacc[db][4 * g] * scale, dkacc[db][4 * g + 1] * scale, dkacc[db][4 * g + 2] * scale,
                            dkacc[db][4 * g + 3] * scale};
                *reinterpret_cast<floatx4*>(vrow + d) =
                    floatx4{dvacc[db][4 * g], dvacc[db][4 * g + 1], dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]};
            }
    }
}

// dQ: one workgroup of 4 waves per (128-query tile, query head); each wave
// owns 32 queries and keeps their Q and dO rows in registers; K and V stream
// through LDS 32 keys at a time.
template <int D, int MASK>
__global__ void __launch_bounds__(256, BwdF32Traits<D>::kWavesPerSimd)
fa2_bwd_dq_f32_kernel(const BwdParams p) {
    using T = BwdF32Traits<D>;
    const float* __restrict__ Q = static_cast<const float*>(p.q);
    const float* __restrict__ K = static_cast<const float*>(p.k);
    const float* __restrict__ V = static_cast<const float*>(p.v);
    const float* __restrict__ dO = static_cast<const float*>(p.dout);
    float* __restrict__ dQ = static_cast<float*>(p.dq);
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

    // query tiles major (heaviest first under a causal mask), heads fastest
    const int bh = blockIdx.x % p.BH;
    int qt = blockIdx.x / p.BH;
    if (MASK == kMaskCausal) qt = p.n_qt - 1 - qt;
    const int bkv = p.G == 1 ? bh : bh / p.G;
    const BwdSeq sq = bwd_seq(p, p.cu_q ? bh / p.H : 0);
    const int M = sq.M, N = sq.N;
    const int64_t qr = q_row0(p, sq, bh), kvr = kv_row0(p, sq, bkv);
    const int qw0 = qt * T::kBlock + 32 * wave;  // first query row of this wave
    const int qw1 = min(qw0 + 32, M) - 1;        // its last row
    const int query = qw0 + l32;                 // this lane's query row

    // Q and dO rows of the lane's query, d half h: B operands of S^T = K Q^T
    // and dP^T = V dO^T; L (log2 units) and Delta of the row
    float qf[T::kHalfD], of[T::kHalfD];
#pragma unroll
    for (int s = 0; s < T::kHalfD; s += 4) {
        floatx4 x = floatx4{0.f, 0.f, 0.f, 0.f}, y = x;
        if (query < M) {
            x = *reinterpret_cast<const floatx4*>(Q + (qr + query) * D + h * T::kHalfD + s);
            y = *reinterpret_cast<const floatx4*>(dO + (qr + query) * D + h * T::kHalfD + s);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            qf[s + u] = x[u];
            of[s + u] = y[u];
        }
    }
    const float l2 = l2_of(query < M ? p.lse[qr + query] : INFINITY);
    const float dl = query < M ? p.delta[qr + query] : 0.f;

    // 32-key tiles [t0, t0 + n_kv): from the first key the workgroup's first
    // row sees to the last key its last row sees; the wave needs [w0, w1)
    constexpr int BN = T::kRows;
    int t0 = 0, n_kv = 0, w0 = 0, w1 = 0;
    {
        const int r0 = qt * T::kBlock, r1 = min(r0 + T::kBlock, M) - 1;
        if (r0 <= r1) {
            const int klo = key_lo<MASK>(p.wl, r0), khi = key_hi<MASK>(p.wr, r1, N);
            if (klo <= khi) {
                t0 = klo / BN;
                n_kv = khi / BN + 1 - t0;
            }
        }
        if (qw0 <= qw1) {
            const int klo = key_lo<MASK>(p.wl, qw0), khi = key_hi<MASK>(p.wr, qw1, N);
            if (klo <= khi) {
                w0 = klo / BN - t0;
                w1 = khi / BN + 1 - t0;
            }
        }
    }
    const int lim_hi = key_hi<MASK>(p.wr, query, N), lim_lo = key_lo<MASK>(p.wl, query);

    floatx16 dqacc[T::kDB];
#pragma unroll
    for (int db = 0; db < T::kDB; ++db) dqacc[db] = floatx16{};

    const float* Kh = K + kvr * D;
    const float* Vh = V + kvr * D;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    F32Stream<D> st;
    st.init(wave, lane);
    int lane_row, lane_xor, col_lane[T::kDB];
    f32_read_lanes<D>(l32, h, lane_row, lane_xor, col_lane);
    // K and V rows of key tile t0 + kt into LDS (rows past N re-read row
    // N-1; those keys are masked)
    auto issue = [&](int kt, char* kdst, char* vdst) __attribute__((always_inline)) {
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BN>(Kh, st.off, wave_u, t0 + kt, N, kdst);
        copy_tile_to_lds<T::kLoadsPerWave, T::kRowBytes, BN>(Vh, st.off, wave_u, t0 + kt, N, vdst);
    };

    auto compute_tile = [&](int kt, const char* ks, const char* vs) __attribute__((always_inline)) {
        if (kt < w0 || kt >= w1) return;
        int lx = lane_xor, cl[T::kDB];
#pragma unroll
        for (int db = 0; db < T::kDB; ++db) cl[db] = col_lane[db];
        opaque_lanes<T::kDB>(lx, cl);
        // S^T = K Q^T, dP^T = V dO^T (rows: the tile's keys, columns: the
        // wave's queries)
        floatx16 sacc = floatx16{}, pacc = floatx16{};
#pragma unroll
        for (int s = 0; s < T::kHalfD; s += 4) {
            const floatx4 ka = f32_row_read<D>(ks, lane_row, lx, s);
            const floatx4 va = f32_row_read<D>(vs, lane_row, lx, s);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[u], qf[s + u], sacc, 0, 0, 0);
                pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(va[u], of[s + u], pacc, 0, 0, 0);
            }
        }
        // keys outside the lane's visible range (past N, causal, window):
        // register r holds key kbase + acc_row(r, h)
        const int kbase = (t0 + kt) * BN;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = kbase + acc_row(r, h);
            if (kk > lim_hi || kk < lim_lo) sacc[r] = -INFINITY;
        }
        // dS^T = P^T (dP^T - Delta), then dQ^T += K^T dS^T: step r contracts
        // the keys whose dS the lane's register r holds
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pv = fast_exp2(fmaf(sacc[r], c_log2, -l2));
            pacc[r] = pv * (pacc[r] - dl);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int db = 0; db < T::kDB; ++db)
                dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(f32_col_read<D>(ks, cl, r, db), pacc[r], dqacc[db], 0, 0, 0);
        }
    };

    // ---- main loop, unrolled by two over the buffer pair (as in dK/dV)
    if (n_kv > 0) issue(0, sK0, sV0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < n_kv; kt += 2) {
        if (kt + 1 < n_kv) issue(kt + 1, sK1, sV1);
        compute_tile(kt, sK0, sV0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 >= n_kv) break;
        if (kt + 2 < n_kv) issue(kt + 2, sK0, sV0);
        compute_tile(kt + 1, sK1, sV1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: dQ = scale dS K; register r of block db holds
    // d = 32 db + acc_row(r, h) of the lane's query
    if (query < M) {
        const float scale = p.scale;
        float* row = dQ + (qr + query) * D;
#pragma unroll
        for (int db = 0; db < T::kDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * db + 8 * g + 4 * h;
                *reinterpret_cast<floatx4*>(row + d) =
                    floatx4{dqacc[db][4 * g] * scale, dqacc[db][4 * g + 1] * scale, dqacc[db][4 * g + 2] * scale,
                            dqacc[db][4 * g + 3] * scale};
            }
    }
}

// ---------------------------------------------------------------------------
// host side: validation, dispatch table, launches
// ---------------------------------------------------------------------------
struct BwdEntry {
    int dtype, D, mask;
    const void* delta;  // Delta kernel (fp32); null: the dQ kernel computes Delta
    const void* dkdv;
    const void* dq;
    int kv_threads, kv_block_n, kv_block_q;  // dK/dV kernel: threads, keys per workgroup, query tile
    int q_threads, q_block_m, q_block_n;     // dQ kernel: threads, queries per workgroup, key tile
    int delta_rows_per_wg;
};

#define BWD_KERNEL(...) reinterpret_cast<const void*>(&__VA_ARGS__)
// D = 64: 4 waves x 32 keys per dK/dV workgroup with K and V in VGPRs, 64-row
// query tiles, two waves per SIMD (measured ~13% faster than the wave-pair
// kernel at this head dim).  D = 128: the wave-pair kernel (K and V in LDS, 8
// waves per 128 keys), since K, V, dK and dV of 32 keys in VGPRs would leave
// room for only one wave per SIMD.
#define BWD_ROW64(E, code, mask)                                                                   \
    {code, 64, mask, nullptr,                                                                     \
     BWD_KERNEL(fa2_bwd_dkdv_kernel<E, 64, 64, 4, 2, mask>),                                     \
     BWD_KERNEL(fa2_bwd_dq_kernel<E, 64, 64, 4, 2, mask>), 256, 128, 64, 256, 128, 64, 4 * 8}
#define BWD_ROW128(E, code, mask)                                                                  \
    {code, 128, mask, nullptr,                                                                    \
     BWD_KERNEL(fa2_bwd_dkdv_pair_kernel<E, 128, mask>),                                         \
     BWD_KERNEL(fa2_bwd_dq_kernel<E, 128, 32, 4, 2, mask>), 512, 128, 64, 256, 128, 32, 4 * 4}
#define BWD_ROWS(E, code, mask) BWD_ROW64(E, code, mask), BWD_ROW128(E, code, mask)
// fp32: 4 waves x 32 keys (dK/dV) or 32 queries (dQ) per workgroup, 32-row
// streamed tiles; the delta kernel covers 64 / (D / 4) rows per wave
#define BWD_ROW_F32(D, mask)                                                                       \
    {FA2_DTYPE_F32, D, mask, BWD_KERNEL(fa2_bwd_delta_f32_kernel<D>),                             \
     BWD_KERNEL(fa2_bwd_dkdv_f32_kernel<D, mask>), BWD_KERNEL(fa2_bwd_dq_f32_kernel<D, mask>),     \
     256, 128, 32, 256, 128, 32, 4 * (256 / D)}
#define BWD_ROWS_F32(mask) BWD_ROW_F32(64, mask), BWD_ROW_F32(128, mask)
const BwdEntry kBwdTable[] = {
    BWD_ROWS(__bf16, FA2_DTYPE_BF16, kMaskNone),   BWD_ROWS(__bf16, FA2_DTYPE_BF16, kMaskCausal),
    BWD_ROWS(__bf16, FA2_DTYPE_BF16, kMaskLocal),  BWD_ROWS(_Float16, FA2_DTYPE_F16, kMaskNone),
    BWD_ROWS(_Float16, FA2_DTYPE_F16, kMaskCausal), BWD_ROWS(_Float16, FA2_DTYPE_F16, kMaskLocal),
    BWD_ROWS_F32(kMaskNone), BWD_ROWS_F32(kMaskCausal), BWD_ROWS_F32(kMaskLocal),
};
#undef BWD_ROWS_F32
#undef BWD_ROW_F32
#undef BWD_ROWS
#undef BWD_ROW64
#undef BWD_ROW128
#undef BWD_KERNEL

const BwdEntry* find_bwd_entry(int dtype, int64_t D, int mask) {
    for (const BwdEntry& t : kBwdTable)
        if (t.dtype == dtype && t.D == D && t.mask == mask) return &t;
    return nullptr;
}

// Checks shared by every backward entry point: scale, flags, dtype, window
// sides, alignment.  The rest (sizes, null pointers, overlaps) depends on the
// layout.
int bwd_common_checks(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* delta, int64_t H, int64_t Hk,
                      float scale, int causal, int64_t wl, int64_t wr, int dtype) {
    if (Hk < 1 || (H > 0 && (Hk > H || H % Hk != 0))) return FA2_ERR_INVALID_ARGUMENT;
    if (dtype != FA2_DTYPE_F32 && dtype != FA2_DTYPE_BF16 && dtype != FA2_DTYPE_F16) return FA2_ERR_INVALID_ARGUMENT;
    if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARGUMENT;
    if (!(scale > 0.f) || !isfinite(scale)) return FA2_ERR_INVALID_ARGUMENT;
    if (wl < -1 || wr < -1) return FA2_ERR_INVALID_ARGUMENT;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(dout, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) ||
        misaligned(lse, 4) || misaligned(delta, 4))
        return FA2_ERR_INVALID_ARGUMENT;
    return FA2_OK;
}

// The outputs (dq, dk, dv, delta) overlap no other buffer.
bool bwd_outputs_overlap(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, size_t q_bytes,
                         size_t kv_bytes, size_t row_bytes) {
    const struct {
        const void* p;
        size_t n;
    } bufs[] = {{dq, q_bytes}, {dk, kv_bytes}, {dv, kv_bytes}, {delta, row_bytes}, {q, q_bytes},
                {k, kv_bytes}, {v, kv_bytes}, {o, q_bytes}, {lse, row_bytes}, {dout, q_bytes}};
    constexpr int kOutputs = 4;
    for (int i = 0; i < kOutputs; ++i)
        for (int j = 0; j < (int)(sizeof(bufs) / sizeof(bufs[0])); ++j)
            if (j != i && overlaps(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n)) return true;
    return false;
}

// The launches.  fp32: Delta over `rows` rows, dK/dV over n_kt key tiles of
// every K/V head, dQ over n_qt query tiles of every query head (the kernel
// view's BH).  16-bit: dQ first, which also stores Delta, then dK/dV.
int bwd_launch(const BwdEntry* e, BwdParams prm, int64_t rows, int64_t n_kt, int64_t n_qt_kv, int64_t n_qt,
               hipStream_t st) {
    hipError_t err = hipSuccess;
    auto launch_dkdv = [&]() {
        if (err != hipSuccess || n_kt * prm.BHk <= 0) return;
        BwdParams a = prm;
        a.n_qt = (int)n_qt_kv;
        void* args[] = {&a};
        err = hipLaunchKernel(e->dkdv, dim3((unsigned)(n_kt * prm.BHk)), dim3(e->kv_threads), args, 0, st);
    };
    auto launch_dq = [&]() {
        if (err != hipSuccess || rows <= 0 || n_qt * prm.BH <= 0) return;
        BwdParams a = prm;
        a.n_qt = (int)n_qt;
        void* args[] = {&a};
        err = hipLaunchKernel(e->dq, dim3((unsigned)(n_qt * prm.BH)), dim3(e->q_threads), args, 0, st);
    };
    if (e->delta) {
        if (rows > 0) {
            const void* o_arg = prm.o;
            const void* do_arg = prm.dout;
            float* d_arg = prm.delta;
            int r = (int)rows;
            void* dargs[] = {(void*)&o_arg, (void*)&do_arg, &d_arg, &r};
            err = hipLaunchKernel(e->delta, dim3((unsigned)ceil_div(rows, e->delta_rows_per_wg)), dim3(256), dargs,
                                  0, st);
        }
        launch_dkdv();
        launch_dq();
    } else {
        launch_dq();
        launch_dkdv();
    }
    return launch_status(err);
}

}  // namespace

extern "C" int fa2_bwd_local(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, float* delta,
                             int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
                             float scale, int causal, int64_t window_left, int64_t window_right,
                             int dtype, void* stream) {
    // ---- argument checks, all before any HIP call
    if (B < 0 || H < 0 || Hk < 1 || M < 0 || N <= 0 || D <= 0) return FA2_ERR_INVALID_ARGUMENT;
    // a pointer may be null only when its buffer holds no element
    const bool q_rows = B > 0 && H > 0 && M > 0, kv_rows = B > 0;
    if (q_rows && (!q || !o || !lse || !dout || !dq || !delta)) return FA2_ERR_INVALID_ARGUMENT;
    if (kv_rows && (!k || !v || !dk || !dv)) return FA2_ERR_INVALID_ARGUMENT;
    const int chk = bwd_common_checks(q, k, v, o, lse, dout, dq, dk, dv, delta, H, Hk, scale, causal,
                                      window_left, window_right, dtype);
    if (chk != FA2_OK) return chk;

    const int64_t kMax = (int64_t)1 << 31;
    if (B > kMax || H > kMax || M >= kMax || N >= kMax) return FA2_ERR_UNSUPPORTED;
    const int64_t BH = B * H, BHk = B * Hk;
    if (M * D >= kMax || N * D >= kMax || BH * M >= kMax || BHk >= kMax) return FA2_ERR_UNSUPPORTED;
    int64_t wl = window_left, wr = window_right;
    const int mask = normalise_window(wl, wr, causal, M, N);
    const BwdEntry* e = find_bwd_entry(dtype, D, mask);
    if (!e) return FA2_ERR_UNSUPPORTED;
    // without a mask the query heads of a K/V head form one row sequence
    const KernelShape ks = kernel_shape(B, H, Hk, M, mask != kMaskNone);
    // every backward kernel copies one head's Q, dO (K, V) tiles through a
    // buffer resource whose byte size, and the tile offsets inside it, are
    // 32-bit
    const int64_t eb = dtype == FA2_DTYPE_F32 ? 4 : 2;
    if (ks.M * D * eb >= kMax || N * D * eb >= kMax) return FA2_ERR_UNSUPPORTED;
    const int64_t n_kt = ceil_div(N, e->kv_block_n);
    const int64_t n_qt = ceil_div(ks.M, e->q_block_m);
    if (n_kt * BHk >= kMax || n_qt * ks.BH >= kMax) return FA2_ERR_UNSUPPORTED;
    const size_t elt = dtype == FA2_DTYPE_F32 ? 4 : 2;
    const size_t q_bytes = (size_t)BH * M * D * elt, kv_bytes = (size_t)BHk * N * D * elt,
                 row_bytes = (size_t)BH * M * 4;
    if (bwd_outputs_overlap(q, k, v, o, lse, dout, dq, dk, dv, delta, q_bytes, kv_bytes, row_bytes))
        return FA2_ERR_INVALID_ARGUMENT;

    if (BHk == 0) return FA2_OK;  // no K/V rows: nothing to write

    BwdParams prm{};  // dense layout: cu_q = cu_k = null
    prm.q = q; prm.k = k; prm.v = v; prm.dout = dout; prm.o = o; prm.lse = lse; prm.delta = delta;
    prm.dq = dq; prm.dk = dk; prm.dv = dv;
    prm.BH = (int)ks.BH;
    prm.BHk = (int)BHk;
    prm.H = (int)ks.H;
    prm.Hk = (int)Hk;
    prm.G = H > 0 ? (int)ks.G : 0;  // no query heads: dK = dV = 0
    prm.M = (int)ks.M;
    prm.N = (int)N;
    prm.wl = (int)wl;
    prm.wr = (int)wr;
    prm.c_log2 = scale * kLog2e;
    prm.scale = scale;
    return bwd_launch(e, prm, BH * M, n_kt, ceil_div(ks.M, e->kv_block_q), n_qt, static_cast<hipStream_t>(stream));
}

extern "C" int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, float* delta,
                       int64_t B, int64_t H, int64_t Hk, int64_t M, int64_t N, int64_t D,
                       float scale, int causal, int dtype, void* stream) {
    return fa2_bwd_local(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Hk, M, N, D, scale, causal, -1, -1,
                         dtype, stream);
}

extern "C" int fa2_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, void* dq, void* dk, void* dv, float* delta,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int64_t B, int64_t H, int64_t Hk, int64_t total_q, int64_t total_k,
                              int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D, float scale, int causal,
                              int64_t window_left, int64_t window_right, int dtype, void* stream) {
    // ---- argument checks, all before any HIP call
    if (B < 0 || H < 0 || Hk < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || D <= 0)
        return FA2_ERR_INVALID_ARGUMENT;
    if (max_seqlen_q > total_q || max_seqlen_k > total_k) return FA2_ERR_INVALID_ARGUMENT;
    if (B > 0 && (!cu_seqlens_q || !cu_seqlens_k)) return FA2_ERR_INVALID_ARGUMENT;
    if (misaligned(cu_seqlens_q, 4) || misaligned(cu_seqlens_k, 4)) return FA2_ERR_INVALID_ARGUMENT;
    if (H > 0 && total_q > 0 && (!q || !o || !lse || !dout || !dq || !delta)) return FA2_ERR_INVALID_ARGUMENT;
    if (total_k > 0 && (!k || !v || !dk || !dv)) return FA2_ERR_INVALID_ARGUMENT;
    const int chk = bwd_common_checks(q, k, v, o, lse, dout, dq, dk, dv, delta, H, Hk, scale, causal,
                                      window_left, window_right, dtype);
    if (chk != FA2_OK) return chk;

    const int64_t kMax = (int64_t)1 << 31;
    // byte offsets inside a head are 32-bit (buffer-resource tile copies)
    const int64_t elt = dtype == FA2_DTYPE_F32 ? 4 : 2;
    if (B >= kMax || H >= kMax || Hk >= kMax || total_q * D * elt >= kMax || total_k * D * elt >= kMax ||
        H * total_q >= kMax)
        return FA2_ERR_UNSUPPORTED;
    int64_t wl = window_left, wr = window_right;
    const int mask = normalise_window(wl, wr, causal, total_q, total_k);
    const BwdEntry* e = find_bwd_entry(dtype, D, mask);
    if (!e) return FA2_ERR_UNSUPPORTED;
    const int64_t BH = B * H, BHk = B * Hk;
    const int64_t n_kt = ceil_div(max_seqlen_k, e->kv_block_n);
    const int64_t n_qt = ceil_div(max_seqlen_q, e->q_block_m);
    if (BH >= kMax || n_kt * BHk >= kMax || n_qt * BH >= kMax) return FA2_ERR_UNSUPPORTED;
    const size_t eb = dtype == FA2_DTYPE_F32 ? 4 : 2;
    const size_t q_bytes = (size_t)H * total_q * D * eb, kv_bytes = (size_t)Hk * total_k * D * eb,
                 row_bytes = (size_t)H * total_q * 4;
    if (bwd_outputs_overlap(q, k, v, o, lse, dout, dq, dk, dv, delta, q_bytes, kv_bytes, row_bytes))
        return FA2_ERR_INVALID_ARGUMENT;

    if (BHk == 0) return FA2_OK;

    BwdParams prm{};
    prm.q = q; prm.k = k; prm.v = v; prm.dout = dout; prm.o = o; prm.lse = lse; prm.delta = delta;
    prm.dq = dq; prm.dk = dk; prm.dv = dv;
    prm.cu_q = cu_seqlens_q;
    prm.cu_k = cu_seqlens_k;
    prm.total_q = (int)total_q;
    prm.total_k = (int)total_k;
    prm.BH = (int)BH;
    prm.BHk = (int)BHk;
    prm.H = (int)H;
    prm.Hk = (int)Hk;
    prm.G = H > 0 ? (int)(H / Hk) : 0;
    prm.wl = (int)wl;
    prm.wr = (int)wr;
    prm.c_log2 = scale * kLog2e;
    prm.scale = scale;
    return bwd_launch(e, prm, H * total_q, n_kt, ceil_div(max_seqlen_q, e->kv_block_q), n_qt,
                      static_cast<hipStream_t>(stream));
}
