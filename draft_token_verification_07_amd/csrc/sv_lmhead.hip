// sv_lmhead.hip -- the fused lm_head -> greedy verification.
//
// The target's logits over the gamma+1 verified positions are the product of
// the last hidden states and the lm_head weight (SSD inference-engine guide,
// sec. 6: compute_logits turns the hidden states into logits, and for the
// EAGLE3 draft head scatters them through d2t; the 2.16x EAGLE blog, sec. 6,
// ties the cost of this classification matmul to the vocabulary).  Greedy
// verification (SSD guide sec. 7, temperature 0) needs only the argmax of each
// row, so the logits are never written: each GEMM tile reduces its rows to a
// (logit, lowest id) maximum in its epilogue.
//
// logits[m][v] = sum_k hidden[m][k] * W[v][k], bfloat16 inputs, float32
// accumulation on the matrix cores (v_mfma_f32_16x16x32_bf16: per lane, A
// holds row l%16 and k 8(l/16)..+7, B column l%16 and the same k, and the
// 16x16 result rows 4(l/16)..+3 of column l%16).  Both matrices are
// k-contiguous.  The block order puts the row tiles that share a weight tile
// on one XCD, so the weights are read from HBM about once.
//
// Epilogue: per row and 128-column key tile, the largest logit and its
// lowest id as one 64-bit key (order-preserving key of the value, then ~id),
// stored per tile.  lmhead_reduce_kernel takes the maximum key of each row
// and publishes the row result, and the sequence step (chain or tree walk)
// of the greedy path follows.
#include "sv_common.h"
#include "sv_internal.h"
#include "sv_rows.h"

namespace sv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kLmThreads = 128 * kLmGroup;      // 2 x kLmGroup waves, each a 64-row x 128-column tile
constexpr int kLmBM = kLmTile;                  // rows per workgroup tile
constexpr int kLmBN = kLmTile * kLmGroup;       // columns per workgroup tile: one key tile per wave column
constexpr int kLmBK = 32;                       // k per stage (one MFMA k)
constexpr int kLmPitch = kLmBK * 2;             // LDS bytes per operand row and stage
constexpr int kLmPA = kLmBM * 4 / kLmThreads;   // 16-byte pieces of A per thread and stage
constexpr int kLmPB = kLmBN * 4 / kLmThreads;   // 16-byte pieces of W per thread and stage
static_assert(kLmThreads / kWave == 2 * kLmGroup, "2 x kLmGroup wave tiles");

// Position of 16-byte piece c of operand row r inside its 64-byte LDS row.
// XOR-ing the piece index with ((r >> 1) ^ (r >> 3)) & 3 makes both access
// patterns touch disjoint banks within each aligned group of 8 lanes (32
// banks of 4 bytes) and within each aligned group of 16 (64 banks): the stage
// writes (consecutive lanes hold the four pieces of consecutive rows, rows
// starting at multiples of 2 and 4) and the fragment reads (consecutive lanes
// hold one piece of consecutive rows, starting at multiples of 16).
__device__ __forceinline__ int lm_piece(int r, int c) { return c ^ (((r >> 1) ^ (r >> 3)) & 3); }

// One stage (32 k) of both operands in registers: thread t holds the pieces
// t, t + kLmThreads, ... of the row-major [row][4 pieces] order, so four
// threads read each row's 64 contiguous bytes.
struct Stage {
    u32x4 a[kLmPA];
    u32x4 b[kLmPB];
    bool kin;     // this thread's pieces lie inside d (else they are stored as zeros)
};

__device__ __forceinline__ void stage_load(Stage &st, const uint16_t *A, const uint16_t *B, int32_t m0, int32_t n0,
                                           int32_t M, int32_t V, int32_t d, int32_t k0) {
    // k past the end (a last stage shorter than 32, or a stage past d) reads
    // the row's last piece and is stored as zeros: the loads themselves are
    // unconditional and in bounds
    const int32_t k = k0 + ((int)threadIdx.x % 4) * 8;
    const int32_t kc = min(k, d - 8);
    st.kin = k < d;
#pragma unroll
    for (int u = 0; u < kLmPA; ++u) {
        const int p = u * kLmThreads + (int)threadIdx.x;
        const int32_t r = min(m0 + p / 4, M - 1);
        st.a[u] = *reinterpret_cast<const u32x4 *>(A + (size_t)r * d + kc);
    }
#pragma unroll
    for (int u = 0; u < kLmPB; ++u) {
        const int p = u * kLmThreads + (int)threadIdx.x;
        const int32_t c = min(n0 + p / 4, V - 1);
        st.b[u] = *reinterpret_cast<const u32x4 *>(B + (size_t)c * d + kc);
    }
}

__device__ __forceinline__ void stage_store(const Stage &st, unsigned char *sa, unsigned char *sb) {
#pragma unroll
    for (int u = 0; u < kLmPA; ++u) {
        const int p = u * kLmThreads + (int)threadIdx.x;
        *reinterpret_cast<u32x4 *>(sa + (p / 4) * kLmPitch + lm_piece(p / 4, p % 4) * 16) =
            st.kin ? st.a[u] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kLmPB; ++u) {
        const int p = u * kLmThreads + (int)threadIdx.x;
        *reinterpret_cast<u32x4 *>(sb + (p / 4) * kLmPitch + lm_piece(p / 4, p % 4) * 16) =
            st.kin ? st.b[u] : u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ bf16x8 frag_a(const unsigned char *sa, int wm, int lr, int lg, int i) {
    const int r = wm * 64 + 16 * i + lr;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sa + r * kLmPitch + lm_piece(r, lg) * 16));
}

__device__ __forceinline__ bf16x8 frag_b(const unsigned char *sb, int wn, int lr, int lg, int j) {
    const int r = wn * kLmTile + 16 * j + lr;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(sb + r * kLmPitch + lm_piece(r, lg) * 16));
}

// A workgroup of eight waves (two per SIMD, one workgroup per CU) computes a
// 128 x 512 tile of logits, each wave 64 x 128 (4 x 8 MFMA tiles, 128
// accumulator registers).  The k loop is software-pipelined, one 32-k stage
// per step:
//  - the A operands of stage s + 1 are read from LDS at the start of step s
//    and each W operand of stage s + 1 right after the MFMAs of its column,
//    so the reads can overlap the matrix cores' work on stage s;
//  - LDS holds stages s and s + 1 (two buffers of 40 KB); stage s + 2 is
//    written to the buffer of stage s once every wave has read it;
//  - the global loads of stage s + 3 are issued right after stage s + 2 is
//    stored and stay in flight across the barrier, which waits for LDS
//    accesses only.
__global__ __launch_bounds__(kLmThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lmhead_kernel(LmheadArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char s_a[2][kLmBM * kLmPitch];
    __shared__ __attribute__((aligned(16))) unsigned char s_b[2][kLmBN * kLmPitch];
    // block -> (row tile, column tile): the row tiles of one column tile on one XCD
    const int32_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int32_t mt = slot % a.mtiles;
    const int32_t ntg = (slot / a.mtiles) * 8 + xcd;            // column tile
    if (ntg * kLmBN >= a.V) return;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int wm = wv / kLmGroup, wn = wv % kLmGroup;
    const int32_t M = a.M, V = a.V, d = a.d;
    const int32_t bm0 = mt * kLmBM, bn0 = ntg * kLmBN;
    const int lr = lane & 15, lg = lane >> 4;
    const int32_t nk = max(2, (d + kLmBK - 1) / kLmBK);   // 32-k stages; a stage past d reads as zeros
    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // MFMA operands of the current stage: A rows wm * 64 + 16 i + (l % 16) and
    // W rows (columns) wn * 128 + 16 j + (l % 16), k 8 (l / 16) .. + 7
    bf16x8 fa[4], fb[8];
    Stage s0;
    stage_load(s0, a.hidden, a.W, bm0, bn0, M, V, d, 0);
    stage_store(s0, s_a[0], s_b[0]);
    stage_load(s0, a.hidden, a.W, bm0, bn0, M, V, d, kLmBK);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag_a(s_a[0], wm, lr, lg, i);
#pragma unroll
    for (int j = 0; j < 8; ++j) fb[j] = frag_b(s_b[0], wn, lr, lg, j);
    stage_store(s0, s_a[1], s_b[1]);
    stage_load(s0, a.hidden, a.W, bm0, bn0, M, V, d, 2 * kLmBK);
    lds_barrier();
    for (int32_t k = 0; k < nk - 1; ++k) {
        // stage k in fa and fb, stage k + 1 in LDS buffer nx, stage k + 2 in s0
        const int nx = (k & 1) ^ 1;
        bf16x8 na[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) na[i] = frag_a(s_a[nx], wm, lr, lg, i);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            fb[j] = frag_b(s_b[nx], wn, lr, lg, j);     // column j's MFMAs are issued: its next operand
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = na[i];
        // every wave read stage k's buffer before the previous barrier
        stage_store(s0, s_a[nx ^ 1], s_b[nx ^ 1]);
        stage_load(s0, a.hidden, a.W, bm0, bn0, M, V, d, (k + 3) * kLmBK);   // may lie past d: zeros
        lds_barrier();
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    // epilogue: per row, the largest logit over this wave's 128 columns (one
    // key tile), lowest id on ties -- per lane over its eight columns, then
    // over the 16 lanes holding the same rows (MFMA result rows 4 (l / 16) + e
    // of column l % 16)
    const int32_t n0 = bn0 + wn * kLmTile;
    const int32_t nt = ntg * kLmGroup + wn;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint64_t best = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t c = n0 + 16 * j + lr;
                const uint64_t key = c < V ? (((uint64_t)zkey(acc[i][j][e]) << 32) | (uint32_t)~(uint32_t)c) : 0ull;
                best = key > best ? key : best;
            }
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) {
                const uint64_t other = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), o, kWave) << 32) |
                                       (uint32_t)__shfl_xor((int)(uint32_t)best, o, kWave);
                best = other > best ? other : best;
            }
            const int32_t r = bm0 + wm * 64 + 16 * i + 4 * lg + e;
            if (lr == 0 && r < M && nt < a.ntiles) a.part[(size_t)r * a.ntiles + nt] = best;
        }
    }
}

// ---------------------------------------------------------------------------
// For d a multiple of 64: the same tiles with 64-k stages copied from global
// memory straight into LDS (global_load_lds_dwordx4: lane i of a wave writes
// 16 bytes at the wave's LDS address + 16 i).  A row segment of a stage is a
// whole 128-byte line, a step carries 64 MFMAs per wave between barriers, and
// no registers stage the data.  Two stages of 80 KB fill the LDS.
// ---------------------------------------------------------------------------
constexpr int kLmBK2 = 64;                                       // k per stage
constexpr int kLmPitch2 = kLmBK2 * 2;                            // LDS bytes per operand row and stage
constexpr int kLmStage2 = (kLmBM + kLmBN) * kLmPitch2;           // A rows, then W rows
constexpr int kLmChunks2 = (kLmBM + kLmBN) / 8;                  // 1 KB chunks (8 rows) per stage
constexpr int kLmChunksPerWave2 = kLmChunks2 / (kLmThreads / kWave);
static_assert(kLmChunks2 % (kLmThreads / kWave) == 0, "whole chunks per wave");
static_assert(2 * kLmStage2 <= 160 * 1024, "two stages fit the LDS");

// Position of 16-byte piece c of row r inside its 128-byte LDS row: the XOR
// with (r & 7) ^ ((r >> 3) & 1) keeps the fragment reads (consecutive lanes
// hold one piece of consecutive rows) free of bank conflicts within each
// aligned group of 8 lanes (32 banks) and of 16 lanes (64 banks).
__device__ __forceinline__ int lm_piece8(int r, int c) { return c ^ ((r & 7) ^ ((r >> 3) & 1)); }

// Stage k0 .. k0 + 63 of both operands into `sbuf`.  Chunk c covers stage rows
// 8 c .. 8 c + 7 (A rows first); lane i fills physical piece i % 8 of row
// i / 8, so it loads the logical piece the swizzle puts there.
__device__ __forceinline__ void stage_dma64(unsigned char *sbuf, const uint16_t *A, const uint16_t *B, int32_t m0,
                                            int32_t n0, int32_t M, int32_t V, int32_t d, int32_t k0, int wv,
                                            int lane) {
#pragma unroll
    for (int q = 0; q < kLmChunksPerWave2; ++q) {
        const int c = wv + q * (kLmThreads / kWave);
        const bool isa = c < kLmBM / 8;                        // alike in the whole wave
        const int r = (isa ? 8 * c : 8 * c - kLmBM) + lane / 8;     // row within A or within the W tile
        const int piece = lm_piece8(r, lane % 8);
        const uint16_t *src = isa ? A + (size_t)min(m0 + r, M - 1) * d : B + (size_t)min(n0 + r, V - 1) * d;
        __builtin_amdgcn_global_load_lds(src + k0 + 8 * piece, sbuf + c * 1024, 16, 0, 0);
    }
}

__device__ __forceinline__ bf16x8 frag_a64(const unsigned char *sa, int wm, int lr, int lg, int i, int h) {
    const int r = wm * 64 + 16 * i + lr;
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const u32x4 *>(sa + r * kLmPitch2 + lm_piece8(r, 4 * h + lg) * 16));
}
__device__ __forceinline__ bf16x8 frag_b64(const unsigned char *sb, int wn, int lr, int lg, int j, int h) {
    const int r = wn * kLmTile + 16 * j + lr;
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const u32x4 *>(sb + r * kLmPitch2 + lm_piece8(r, 4 * h + lg) * 16));
}

__global__ __launch_bounds__(kLmThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lmhead_dma_kernel(
    LmheadArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char s_st[2][kLmStage2];
    const int32_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int32_t mt = slot % a.mtiles;
    const int32_t ntg = (slot / a.mtiles) * 8 + xcd;            // column tile
    if (ntg * kLmBN >= a.V) return;
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int wm = wv / kLmGroup, wn = wv % kLmGroup;
    const int32_t M = a.M, V = a.V, d = a.d;
    const int32_t bm0 = mt * kLmBM, bn0 = ntg * kLmBN;
    const int lr = lane & 15, lg = lane >> 4;
    const int32_t nk = d / kLmBK2;                              // >= 1
    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto dma = [&](int32_t s) {
        stage_dma64(s_st[s & 1], a.hidden, a.W, bm0, bn0, M, V, d, s * kLmBK2, wv, lane);
    };
    dma(0);
    if (nk > 1) {
        dma(1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLmChunksPerWave2) : "memory");   // stage 0 landed (this wave)
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();
    bf16x8 fa[4], fb[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag_a64(s_st[0], wm, lr, lg, i, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) fb[j] = frag_b64(s_st[0] + kLmBM * kLmPitch2, wn, lr, lg, j, 0);
    for (int32_t k = 0; k < nk; ++k) {
        // stage k's first half in fa / fb; stage k + 1 in flight into the other
        // buffer (issued here from k = 1 on: that buffer's stage k - 1 was read
        // before the last barrier)
        if (k >= 1 && k + 1 < nk) dma(k + 1);
        const unsigned char *sa = s_st[k & 1];
        const unsigned char *sb = sa + kLmBM * kLmPitch2;
        // first half: its MFMAs, with the second half's operands read meanwhile
        bf16x8 na[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) na[i] = frag_a64(sa, wm, lr, lg, i, 1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            fb[j] = frag_b64(sb, wn, lr, lg, j, 1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = na[i];
        // second half
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        if (k + 1 < nk) {
            // stage k + 1 landed (this wave's loads, then everyone's), then its first half
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            const unsigned char *na2 = s_st[(k + 1) & 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = frag_a64(na2, wm, lr, lg, i, 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) fb[j] = frag_b64(na2 + kLmBM * kLmPitch2, wn, lr, lg, j, 0);
        }
    }
    // epilogue as in lmhead_kernel
    const int32_t n0 = bn0 + wn * kLmTile;
    const int32_t nt = ntg * kLmGroup + wn;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint64_t best = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t c = n0 + 16 * j + lr;
                const uint64_t key = c < V ? (((uint64_t)zkey(acc[i][j][e]) << 32) | (uint32_t)~(uint32_t)c) : 0ull;
                best = key > best ? key : best;
            }
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) {
                const uint64_t other = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), o, kWave) << 32) |
                                       (uint32_t)__shfl_xor((int)(uint32_t)best, o, kWave);
                best = other > best ? other : best;
            }
            const int32_t r = bm0 + wm * 64 + 16 * i + 4 * lg + e;
            if (lr == 0 && r < M && nt < a.ntiles) a.part[(size_t)r * a.ntiles + nt] = best;
        }
    }
}

// One wave per row: the maximum key over the row's column tiles, published
// as the row result (value, id); optionally written out.
__global__ __launch_bounds__(256) void lmhead_reduce_kernel(LmheadArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int32_t r = blockIdx.x * 4 + (int32_t)(threadIdx.x / kWave);
    if (r >= a.M) return;
    const uint64_t *p = a.part + (size_t)r * a.ntiles;
    uint64_t best = 0;
    for (int32_t c = lane; c < a.ntiles; c += kWave) best = p[c] > best ? p[c] : best;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t other = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), o, kWave) << 32) |
                               (uint32_t)__shfl_xor((int)(uint32_t)best, o, kWave);
        best = other > best ? other : best;
    }
    if (lane == 0) {
        ArgMax m;
        m.v = fkey_inv((uint32_t)(best >> 32));
        m.i = (int32_t)~(uint32_t)best;
        pub(&a.rowres[r], m);
        if (a.out_argmax) a.out_argmax[r] = m.i;
        if (a.out_maxlogit) a.out_maxlogit[r] = m.v;
    }
}

hipError_t launch_lmhead(const LmheadArgs &a, hipStream_t st) {
    const int64_t grid = (int64_t)a.mtiles * a.ntiles8;
#ifndef SV_LM_DMA
#define SV_LM_DMA 1
#endif
    if (SV_LM_DMA && a.d % kLmBK2 == 0)
        hipLaunchKernelGGL(lmhead_dma_kernel, dim3((unsigned)grid), dim3(kLmThreads), 0, st, a);
    else
        hipLaunchKernelGGL(lmhead_kernel, dim3((unsigned)grid), dim3(kLmThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_reduce_kernel, dim3((unsigned)((a.M + 3) / 4)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace sv
