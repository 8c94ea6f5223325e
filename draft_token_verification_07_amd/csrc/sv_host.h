// sv_host.h -- the host-side parts of the library that need no GPU: launch
// tuning, the plain-data argument blocks shared with the kernels, workspace
// geometry and the argument checks of the C ABI.  Plain C++17 (the HIP
// runtime API header supplies the public stream type); the kernels see it
// through sv_internal.h.  Not installed.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

// (value, id) of a row or chunk maximum; ties keep the lowest id
struct ArgMax {
    float v;
    int32_t i;
};
// online softmax statistics: maximum and sum of 2^((z - m) c)
struct MaxSum {
    float m;
    float s;
};

// ---------------------------------------------------------------------------
// Tuning (chosen by measurement on MI355X; see the design notes).
// ---------------------------------------------------------------------------
#ifndef SV_GREEDY_THREADS
#define SV_GREEDY_THREADS 256
#endif
#ifndef SV_GREEDY_UNROLL
#define SV_GREEDY_UNROLL 4
#endif
#ifndef SV_GREEDY_ITERS
#define SV_GREEDY_ITERS 16
#endif
#ifndef SV_GREEDY_WIDE
#define SV_GREEDY_WIDE 2
#endif
#ifndef SV_GREEDY_MIN_WGS
#define SV_GREEDY_MIN_WGS 256
#endif
#ifndef SV_STATS_THREADS
#define SV_STATS_THREADS 256
#endif
#ifndef SV_STATS_UNROLL
#define SV_STATS_UNROLL 4
#endif
#ifndef SV_STATS_ITERS
#define SV_STATS_ITERS 4
#endif
#ifndef SV_TOPP_THREADS
#define SV_TOPP_THREADS 512
#endif
#ifndef SV_TOPP_UNROLL
#define SV_TOPP_UNROLL 4
#endif

constexpr int kGreedyThreads = SV_GREEDY_THREADS;
constexpr int kGreedyUnroll = SV_GREEDY_UNROLL;
constexpr int kGreedyItersPerWg = SV_GREEDY_ITERS;
constexpr int kGreedyMinWgs = SV_GREEDY_MIN_WGS;    // rows are cut until the grid has this many
constexpr int kGreedyWideMaxWgs = 512;              // grids this small take SV_GREEDY_WIDE * kGreedyThreads per workgroup
constexpr int kGreedyMinChunkVecs = 1024;           // ... but chunks keep this many 16-byte vectors
#ifndef SV_ROW_GROUP
#define SV_ROW_GROUP 8
#endif
constexpr int kRowGroup = SV_ROW_GROUP;             // longer sequences end the row launch and walk in a second
constexpr int kStatsThreads = SV_STATS_THREADS;     // plain-mode row statistics
constexpr int kStatsUnroll = SV_STATS_UNROLL;
constexpr int kStatsItersPerWg = SV_STATS_ITERS;
constexpr int kToppThreads = SV_TOPP_THREADS;       // one workgroup per row with top-p
constexpr int kToppUnroll = SV_TOPP_UNROLL;
constexpr int kSampThreads = 256;                   // residual / bonus draw
constexpr int kMaxChunks = 4096;

// Top-p band: during streaming a 16-byte vector is copied to LDS when its
// largest logit is within kToppBandNats * T of the running row maximum (so
// y = z / T is within kToppBandNats of max y); afterwards the band is the set
// of tokens within that distance of the final maximum.  The band is checked
// to hold more than top_p of the row's mass; otherwise the row takes the
// exact radix-select path over the whole row.
constexpr float kToppBandNats = 8.0f;
constexpr int kCandCap = 2048;      // LDS slots for band tokens per row
constexpr int kCandVecCap = 1024;   // LDS slots for band vectors (16 bytes each) per row
constexpr int kKeptCap = 2048;      // kept-list entries stored per row
constexpr int kQListCap = 1024;     // q lists up to this size are matched in LDS during a draw
#ifndef SV_TILE
#define SV_TILE 2048
#endif
constexpr int kTile = SV_TILE;      // most target ids per residual/bonus tile
constexpr int kTileMin = 1024;      // fewest (tiles shrink for small batches)
constexpr int kSubTiles = 64;       // equal id ranges per tile whose masses the pick reads
constexpr int kDrawMinWgs = 512;    // tiles shrink until the draw has this many workgroups
#ifndef SV_STATS_MIN_WGS
#define SV_STATS_MIN_WGS 256
#endif
constexpr int kStatsMinWgs = SV_STATS_MIN_WGS;  // plain-mode chunks shrink until the grid has this many (small batches)
constexpr int kStatsMinChunk = 2048;  // ... but never below this many elements per chunk
#ifndef SV_STATS_CHUNK_BYTES
#define SV_STATS_CHUNK_BYTES 131072
#endif
constexpr int kStatsChunkBytes = SV_STATS_CHUNK_BYTES;  // logits bytes per plain-mode chunk
constexpr int kPartCap = 2048;      // chunk partials staged in LDS by a sequence epilogue

// ---------------------------------------------------------------------------
// Greedy / tree
// ---------------------------------------------------------------------------
struct GreedyArgs {
    const void *logits;
    const int32_t *tokens;     // chain: [B, gamma]; tree: [B, N]
    const int32_t *parents;    // tree only: [B, N]
    int32_t B, rows_per_seq, V, chunks;
    int32_t tree;
    int32_t split_chunks;      // the sequence launch merges chunk results (split launch, chunks > 1)
    int32_t *out_tokens, *out_len, *out_status, *out_path;
    ArgMax *part;              // [B * rows_per_seq * chunks] chunk results (chunks > 1)
    ArgMax *rowres;            // [B * rows_per_seq] row results
    uint32_t *counters;        // [B] sequences (single-launch path)
};

int32_t greedy_chunks(int32_t V, int64_t rows);
bool greedy_split(int32_t R, int32_t C);

// ---------------------------------------------------------------------------
// Fused lm_head -> greedy verification
// ---------------------------------------------------------------------------
struct LmheadArgs {
    const uint16_t *hidden;     // [M, d] bfloat16 bits, M = B * R
    const uint16_t *W;          // [V, d] bfloat16 bits
    int32_t M, d, V;
    int32_t mtiles, ntiles, ntiles8;   // 128-row / 128-column tiles; ntiles8: GEMM column tiles rounded up to 8
    uint64_t *part;             // [M, ntiles] (value, ~id) max-keys per row and column tile
    ArgMax *rowres;             // [M] published row results
    int32_t *out_argmax;        // [M] or null
    float *out_maxlogit;        // [M] or null
};
constexpr int kLmTile = 128;      // rows per GEMM row tile, columns per key tile
constexpr int kLmGroup = 4;       // key tiles per GEMM column tile (512 columns)

// ---------------------------------------------------------------------------
// Sampling
// ---------------------------------------------------------------------------

// Per-row distribution descriptor.  Token id j of the row (own vocabulary)
// with logit z has weight w = 2^((z - m) * c), c = log2(e) / T.  It is kept
// iff key(z) > key || (key(z) == key && j <= tie_cut), where key() is the
// order-preserving key of z with -0 folded onto +0; without top-p key = 0 and
// tie_cut = INT32_MAX keep every id.  p(j) = w / Zk for kept ids, else 0.
struct RowDesc {
    float m;          // row maximum of the raw logits
    float Z;          // sum of w over the whole row
    float Zk;         // sum of w over the kept ids
    uint32_t key;
    int32_t tie_cut;
    int32_t nkept;    // kept ids; the list is stored iff nkept <= kKeptCap
    int32_t flags;    // RD_* bits
    float ptok;       // p (or q) of the row's draft token; 0 for the bonus row
};
enum { RD_NO_MASS = 1, RD_HAS_LIST = 2, RD_FALLBACK = 4, RD_BAD_MAP = 8 };

struct KeptEnt {      // one kept id of a row and its weight w
    int32_t id;
    float w;
};

struct Probe {        // the logits at one draft token: target row, draft row
    float zt;         // target logit of x_i (0 when x_i is out of range)
    float zd;         // draft logit of x_i; -inf when x_i is off the d2t map
};

struct SeqState {     // written by the statistics epilogue for the draw kernel
    int32_t n;        // accepted drafts
    int32_t status;   // SV_SEQ_* bits
    int32_t pad0, pad1;
    RowDesc dp, dq;   // the rows the draw uses: target row n, draft row n (= dp for the bonus)
};

struct SampleArgs {
    const void *tl;            // target logits [B, gamma+1, Vt]
    const void *dl;            // draft logits  [B, gamma, Vd]
    const int32_t *tokens;     // [B, gamma]
    const int32_t *d2t;        // [Vd] or null
    const float *u_acc;        // [B, gamma]
    const float *u_s;          // [B]
    int32_t B, gamma, Vt, Vd;
    float T, c, top_p;         // c = log2(e) / T
    int32_t topp;              // top-p filter on
    int32_t Ct, Cd;            // chunks per target / draft row (1 with top-p)
    int32_t tile, ntiles;      // target ids per draw tile, draw tiles per row
    int32_t *out_tokens, *out_len, *out_status;
    float *out_p, *out_q;
    // workspace
    uint32_t *cnt_stats;       // [B] (top-p)
    uint32_t *map_flag;        // [1] after cnt_stats: nonzero once a plain-mode call sees a bad d2t map
                               // (set by the probe workgroups, read by the draw tiles, cleared by the pick)
    SeqState *seq;             // [B]
    RowDesc *rows;             // [B, 2*gamma+1]: target rows then draft rows
    MaxSum *part;              // [B, (gamma+1)*Ct + gamma*Cd]
    KeptEnt *kept;             // [B, 2*gamma+1, kept_stride] (top-p only)
    int32_t kept_stride;       // min(kKeptCap, max(Vt, Vd))
    Probe *probe;              // [B, gamma] (plain mode)
    uint64_t *tile_mass;       // [B, ntiles] fixed-point draw masses (plain mode)
    uint64_t *tile_sub;        // [B, ntiles, kSubTiles] the same by subtile (plain mode)
    int32_t *tile_jb;          // [ntiles + 1] first draft id of each draw tile under d2t (plain mode)
};

// ---------------------------------------------------------------------------
// Draft-side sampler
// ---------------------------------------------------------------------------
struct ChunkRes {     // one chunk of a draft row: online (max, sum) and its band
    float m, s;
    int32_t n;        // band tokens published (<= kCandCap), -1 when the band overflowed
    int32_t pad;
};

struct DraftArgs {
    const void *logits;        // [B, V]
    const int32_t *d2t;        // [V] or null: report target id d2t[j] for draft id j
    const float *u;            // [B]
    int32_t B, V, C;           // C chunks per row
    float T, c, top_p;         // c = log2(e) / T
    int32_t top_k;             // 0 = off
    int32_t *out_tokens;
    float *out_prob;
    int32_t *out_status;
    // workspace
    uint32_t *counters;        // [B] arrivals
    ChunkRes *res;             // [B, C]
    uint64_t *cand;            // [B, C, kCandCap] ordering codes of band tokens
    RowDesc *desc;             // [B] (exact fallback)
};
struct DraftLayout {
    size_t counter_bytes;
    size_t res, cand, desc, data_bytes;   // offsets from K
};
constexpr int kDraftMaxChunks = 8;
constexpr int kDraftMinChunk = 8192;       // logits per chunk at least
constexpr int kDraftTargetWgs = 256;       // chunks grow until the grid has about this many workgroups
int32_t draft_chunks(int32_t B, int32_t V);
void draft_layout(int32_t B, int32_t V, DraftLayout *L, int32_t *C);

// ---------------------------------------------------------------------------
// SSD fan-out lookup
// ---------------------------------------------------------------------------
struct FanoutArgs {
    const int32_t *out_tokens;   // [B, gamma+1]
    const int32_t *accept_len;   // [B]
    const int32_t *cand;         // [B, gamma+1, f]
    const int32_t *drafts;       // [B, (gamma+1) f, L] (may be null when out_next is)
    int64_t B;
    int32_t gamma, f, L;
    int32_t *out_branch;         // [B]
    int32_t *out_next;           // [B, L] or null
    unsigned long long *counters;  // [2] or null: lookups, hits
};

// ---------------------------------------------------------------------------
// Vocabulary-trim d2t builder
// ---------------------------------------------------------------------------
// State of one call, written by the reduce and refine launches and read by
// the later ones (data region).
struct TrimState {
    unsigned long long valid, invalid;   // tokens in [0, Vt) and outside it
    unsigned long long aboveB;           // mass of the buckets above the boundary bucket
    unsigned long long above;            // mass of the ids with count > cstar
    double T;                            // P * valid
    int32_t mode;                        // 0: nothing kept, 1: every nonzero id, 2: a cut
    int32_t refine;                      // 0: cstar known, 1: exact histogram, 2: sorted list
    uint32_t lo, hi;                     // count range of the boundary bucket
    uint32_t nB;                         // ids in the boundary bucket
    uint32_t cstar, take;                // the cut: ids of count > cstar, and the take lowest of cstar
    uint32_t list_n;                     // entries of the list (refine 2)
};
struct TrimArgs {
    const int32_t *tokens;        // [N]
    int64_t N;
    int32_t Vt;
    float P;
    int32_t *out_d2t;             // [Vt]: the kept ids ascending in the first *out_vd entries
    int32_t *out_t2d;             // [Vt] or null
    int32_t *out_vd;              // [1]
    int64_t *out_info;            // [3] or null: kept mass, valid tokens, invalid tokens
    int32_t S;                    // stream slices
    int32_t R, logR, KB;          // id ranges (ids t with t % R == r), bins per range (a multiple of 8)
    int32_t nblocks;              // 1024-id blocks of the output pass
    uint32_t *part;               // [S, R, KB / 2] partial histograms, two 16-bit bins per word
    uint32_t *ovf;                // [Vt] counts moved out of 16-bit bins (counter region; returned to zero)
    uint32_t *counts;             // [Vt]
    uint32_t *hist_n;             // [kTrimBuckets] ids per count bucket
    unsigned long long *hist_m;   // [kTrimBuckets] their count sum
    uint32_t *h2;                 // [kTrimFine] ids per exact count inside the boundary bucket
    uint32_t *list;               // [kTrimList] counts inside the boundary bucket (wide buckets)
    uint32_t *blockdef, *blocktie;  // [nblocks] ids above the cut / on it, per block
    TrimState *state;
    unsigned long long *totals;   // [0]: valid tokens (counter region; returned to zero); [1] unused
    uint32_t *arrive;             // [2] arrival counters (counter region; returned to zero)
};
constexpr int kTrimBins = 65536;        // 16-bit bins per partial-histogram workgroup (128 KiB of LDS)
constexpr int kTrimTargetWgs = 256;     // ranges x slices
constexpr int kTrimMaxSlices = 128;
constexpr int kTrimBuckets = 1728;      // count buckets: exact below 128, then 64 per octave
constexpr int kTrimFine = 4096;         // widest boundary bucket refined by an exact histogram
constexpr int kTrimList = 4096;         // most ids in a wider boundary bucket
constexpr int kTrimBlock = 1024;        // ids per block of the output pass
size_t trim_counter_bytes(int32_t Vt);
size_t trim_data_bytes(int32_t Vt);
// Fills the size fields and workspace pointers of a (counter region at
// base, data region at data).
void trim_layout(TrimArgs &a, char *base, char *data);

// Workspace of W bytes: [0, K) holds the arrival counters, [K, W) the data,
// with K = counter_region(W) -- a function of W alone.  Every call returns
// its counters to zero, and no call ever writes data below K, so calls of any
// entry point and any size can share one workspace as long as they pass the
// same W (the memory is zeroed once when allocated).
inline size_t counter_region(size_t W) { return (W / 8) & ~(size_t)255; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// Smallest W (a multiple of 256) that fits counter_bytes below K and
// data_bytes above it.
inline size_t workspace_need(size_t counter_bytes, size_t data_bytes) {
    size_t W = align256(8 * counter_bytes + data_bytes + data_bytes / 4 + 4096);
    while (counter_region(W) < counter_bytes || W - counter_region(W) < data_bytes) W += 256;
    return W;
}
inline bool workspace_fits(size_t W, size_t counter_bytes, size_t data_bytes) {
    return counter_region(W) >= counter_bytes && W - counter_region(W) >= data_bytes;
}

struct WorkspaceLayout {
    size_t cnt_stats, counter_bytes;                         // offsets from 0
    size_t seq, rows, part, kept, probe, tile_mass, tile_sub, tile_jb, data_bytes;   // offsets from K
};
// Workspace layout and launch shape of one sampling call; bt / bd are the
// element sizes of the target / draft logits.  4-byte elements give the
// largest layout, which the workspace size query assumes.
bool sample_layout(int32_t B, int32_t gamma, int32_t Vt, int32_t Vd, int32_t bt, int32_t bd, bool topp,
                   WorkspaceLayout *L, int32_t *Ct, int32_t *Cd, int32_t *tile, int32_t *ntiles);
int32_t kept_stride(int32_t Vt, int32_t Vd);

// ---------------------------------------------------------------------------
// Argument checks and sizes of the C ABI (sv_host.cpp)
// ---------------------------------------------------------------------------
bool dtype_ok(int dt);
size_t esize(int dt);
bool aligned(const void *p, size_t a);
bool grid_fits(int64_t wgs);            // the whole grid fits one launch dimension
int32_t greedy_C(int32_t B, int32_t R, int32_t V);
size_t greedy_counter_bytes(int32_t B, int32_t R, int32_t V);
size_t greedy_rowres_bytes(int32_t B, int32_t R);
size_t greedy_data_bytes(int32_t B, int32_t R, int32_t V);
size_t greedy_ws(int32_t B, int32_t R, int32_t V);
int64_t chunk_total_bound(int64_t rows, int64_t c0, int64_t cap, int64_t target, int64_t maxc);
size_t lmhead_part_bytes(int64_t M, int32_t V);
size_t lmhead_data_bytes(int64_t M, int32_t V);
int64_t lmhead_col_tiles8(int32_t V);

// Each check takes an entry point's arguments in the order its declaration
// documents the failures.  It returns the call's status when the host
// decides it -- an error, or SV_OK with nothing to launch (B == 0) -- with
// *launch false; otherwise SV_OK with *launch true and, where given, the
// layout the launch uses.
sv_status check_greedy(const void *target_logits, int dtype, const int32_t *draft_tokens, int32_t B, int32_t gamma,
                       int32_t V, const int32_t *out_tokens, const int32_t *out_accept_len, const void *workspace,
                       size_t workspace_bytes, bool *launch);
sv_status check_tree(const void *target_logits, int dtype, const int32_t *node_tokens, const int32_t *parents,
                     int32_t B, int32_t N, int32_t V, const int32_t *out_path_nodes, const int32_t *out_tokens,
                     const int32_t *out_accept_len, const void *workspace, size_t workspace_bytes, bool *launch);
sv_status check_sample(const void *target_logits, int target_dtype, const void *draft_logits, int draft_dtype,
                       const int32_t *draft_tokens, const int32_t *d2t, const float *u_accept, const float *u_sample,
                       int32_t B, int32_t gamma, int32_t Vt, int32_t Vd, float temperature, float top_p,
                       const int32_t *out_tokens, const int32_t *out_accept_len, const void *workspace,
                       size_t workspace_bytes, WorkspaceLayout *L, int32_t *Ct, int32_t *Cd, int32_t *tile,
                       int32_t *ntiles, bool *launch);
sv_status check_draft(const void *logits, int dtype, const float *u, int32_t B, int32_t V, float temperature,
                      float top_p, const int32_t *out_tokens, const void *workspace, size_t workspace_bytes,
                      DraftLayout *L, int32_t *C, bool *launch);
sv_status check_count(const int32_t *accept_len, int32_t B, int32_t gamma, const uint64_t *counters, bool *launch);
sv_status check_fanout(const int32_t *out_tokens, const int32_t *accept_len, const int32_t *cand,
                       const int32_t *branch_drafts, int32_t B, int32_t gamma, int32_t f, int32_t L,
                       const int32_t *out_branch, const int32_t *out_next, const uint64_t *counters, bool *launch);
sv_status check_trim(const int32_t *tokens, int64_t N, int32_t Vt, float P, const int32_t *out_d2t,
                     const int32_t *out_vd, const int64_t *out_info, const void *workspace, size_t workspace_bytes,
                     bool *launch);
// lm_head chain (tree false, R = gamma + 1, tokens = draft tokens) or tree
// (tree true, R = N, tokens = node tokens)
sv_status check_lmhead(const void *hidden, const void *W, const int32_t *tokens, const int32_t *parents, bool tree,
                       int32_t B, int32_t R, int32_t d, int32_t V, const int32_t *out_path_nodes,
                       const int32_t *out_tokens, const int32_t *out_accept_len, const void *workspace,
                       size_t workspace_bytes, bool *launch);

}  // namespace sv
