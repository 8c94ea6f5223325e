// sv_host.cpp -- the host-side parts of the C ABI that need no GPU:
// workspace geometry of every path, the argument checks of every entry
// point, and the entry points that only compute sizes or strings.  Plain
// C++17; the kernels and launches live in the .hip sources, and the entry
// points there run these checks before any launch.
#include <math.h>

#include "sv_host.h"

namespace sv {

bool dtype_ok(int dt) { return dt == SV_F32 || dt == SV_BF16; }
size_t esize(int dt) { return dt == SV_BF16 ? 2 : 4; }
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool grid_fits(int64_t wgs) { return wgs >= 0 && wgs <= (int64_t)INT32_MAX; }

// Rows are cut into C = min(maxc, max(c0, min(ceil(target / rows), cap)))
// chunks each (c0 and cap grow with the row length): small batches are cut
// further until the grid has about `target` workgroups.  rows * C can then
// fall as rows grows, so buffers of chunk results are sized by this bound
// instead, which never decreases as rows or the row length grow (a workspace
// sized for the largest call serves every smaller one):
//   rows * C <= min(rows * maxc, max(rows * c0, min(rows * cap, target + rows))).
int64_t chunk_total_bound(int64_t rows, int64_t c0, int64_t cap, int64_t target, int64_t maxc) {
    if (rows <= 0) return 0;
    if (c0 < 1) c0 = 1;
    if (cap < 1) cap = 1;
    int64_t b = rows * cap < target + rows ? rows * cap : target + rows;
    if (rows * c0 > b) b = rows * c0;
    return rows * maxc < b ? rows * maxc : b;
}

// ---------------------------------------------------------------------------
// Greedy / tree
// ---------------------------------------------------------------------------
bool greedy_split(int32_t R, int32_t C) { return R > kRowGroup || C > 1; }

// Chunks per row.  Counted in 8-element vectors whatever the dtype, so the
// workspace size depends on V and the row count only (a float32 chunk is
// twice the bytes).  Rows are cut further, down to kGreedyMinChunkVecs
// vectors, while the grid has fewer than kGreedyMinWgs workgroups.
int32_t greedy_chunks(int32_t V, int64_t rows) {
    const int64_t nvec = ((int64_t)V + 7) / 8;
    const int64_t target = (int64_t)kGreedyThreads * kGreedyUnroll * kGreedyItersPerWg;
    int64_t C = (nvec + target - 1) / target;
    const int64_t want = (kGreedyMinWgs + rows - 1) / (rows > 0 ? rows : 1);
    int64_t cap = nvec / kGreedyMinChunkVecs;
    if (cap < 1) cap = 1;
    const int64_t extra = want < cap ? want : cap;
    if (extra > C) C = extra;
    if (C < 1) C = 1;
    if (C > kMaxChunks) C = kMaxChunks;
    return (int32_t)C;
}

// counters [B] (+ [B, R] when rows are chunked) below K; (value, index) row
// results [B, R] and chunk partials [B, R, C] above
int32_t greedy_C(int32_t B, int32_t R, int32_t V) { return greedy_chunks(V, (int64_t)B * R); }
size_t greedy_counter_bytes(int32_t B, int32_t R, int32_t V) {
    const int32_t C = greedy_C(B, R, V);
    return align256(sizeof(uint32_t) * (size_t)B * (C > 1 && !greedy_split(R, C) ? 1 + (size_t)R : 1));
}
size_t greedy_rowres_bytes(int32_t B, int32_t R) { return align256(sizeof(ArgMax) * (size_t)B * R); }
size_t greedy_data_bytes(int32_t B, int32_t R, int32_t V) {
    const int64_t nvec = ((int64_t)V + 7) / 8;
    const int64_t per = (int64_t)kGreedyThreads * kGreedyUnroll * kGreedyItersPerWg;
    const int64_t parts = chunk_total_bound((int64_t)B * R, (nvec + per - 1) / per, nvec / kGreedyMinChunkVecs,
                                            kGreedyMinWgs, kMaxChunks);
    return greedy_rowres_bytes(B, R) + align256(sizeof(ArgMax) * (size_t)parts);
}
size_t greedy_ws(int32_t B, int32_t R, int32_t V) {
    return workspace_need(greedy_counter_bytes(B, R, V), greedy_data_bytes(B, R, V));
}

// ---------------------------------------------------------------------------
// Sampling
// ---------------------------------------------------------------------------
// Chunks per row in plain mode: about 64 KiB of logits each, cut further
// (down to kStatsMinChunk elements) while the grid has fewer than
// kStatsMinWgs workgroups.  A function of the row length, element size and row
// count only, so rows of equal length and type are cut the same way
// (identical rows give identical statistics).
int32_t plain_chunks(int32_t V, int32_t ebytes, int64_t rows) {
    const int64_t per = (int64_t)kStatsChunkBytes / ebytes;
    int64_t C = ((int64_t)V + per - 1) / per;
    const int64_t want = (kStatsMinWgs + rows - 1) / (rows > 0 ? rows : 1);
    int64_t cap = (int64_t)V / kStatsMinChunk;
    if (cap < 1) cap = 1;
    const int64_t extra = want < cap ? want : cap;
    if (extra > C) C = extra;
    if (C < 1) C = 1;
    if (C > kMaxChunks) C = kMaxChunks;
    return (int32_t)C;
}

// Target ids per draw tile: kTile, halved (down to kTileMin) until the draw
// has kDrawMinWgs workgroups.
int32_t draw_tile(int32_t B, int32_t Vt) {
    int32_t tl = kTile;
    while (tl > kTileMin && (int64_t)B * ((Vt + tl - 1) / tl) < kDrawMinWgs) tl >>= 1;
    return tl;
}

// Kept-list slots per row: a row keeps at most as many ids as it has.
int32_t kept_stride(int32_t Vt, int32_t Vd) {
    const int32_t v = Vt > Vd ? Vt : Vd;
    return v < kKeptCap ? v : kKeptCap;
}

bool sample_layout(int32_t B, int32_t gamma, int32_t Vt, int32_t Vd, int32_t bt, int32_t bd, bool topp,
                   WorkspaceLayout *L, int32_t *Ct, int32_t *Cd, int32_t *tile, int32_t *ntiles) {
    const size_t NR = (size_t)(2 * gamma + 1);
    const int32_t ct = topp ? 1 : plain_chunks(Vt, bt, (int64_t)B * (int64_t)NR);
    const int32_t cd = topp ? 1 : plain_chunks(Vd, bd, (int64_t)B * (int64_t)NR);
    const int32_t tl = draw_tile(B, Vt);
    const int32_t nt = (Vt + tl - 1) / tl;
    // Buffers of chunk results and draw tiles are sized by bounds that never
    // decrease as B, gamma or the row lengths grow: the chunk bound with the
    // B (gamma + 1) target rows (B gamma draft rows) as the row count (the
    // chunks are cut for B (2 gamma + 1) rows, so at most as finely), and
    // the tiles at their smallest size.
    const int64_t pt = topp ? 0
                            : chunk_total_bound((int64_t)B * (gamma + 1), ((int64_t)Vt + kStatsChunkBytes / bt - 1) /
                                                    (kStatsChunkBytes / bt), (int64_t)Vt / kStatsMinChunk,
                                                kStatsMinWgs, kMaxChunks);
    const int64_t pd = topp ? 0
                            : chunk_total_bound((int64_t)B * gamma, ((int64_t)Vd + kStatsChunkBytes / bd - 1) /
                                                    (kStatsChunkBytes / bd), (int64_t)Vd / kStatsMinChunk,
                                                kStatsMinWgs, kMaxChunks);
    const size_t ntb = ((size_t)Vt + kTileMin - 1) / kTileMin;      // >= nt
    L->cnt_stats = 0;
    L->counter_bytes = align256(sizeof(uint32_t) * ((size_t)B + 1));     // arrival counters, then the map flag
    size_t off = 0;
    L->seq = off;       off = align256(off + sizeof(SeqState) * (size_t)B);
    L->rows = off;      off = align256(off + sizeof(RowDesc) * (size_t)B * NR);
    L->part = off;      off = align256(off + sizeof(MaxSum) * (size_t)(pt + pd));
    L->kept = off;      off = align256(off + (topp ? sizeof(KeptEnt) * (size_t)B * NR * kept_stride(Vt, Vd) : 0));
    L->probe = off;     off = align256(off + (topp ? 0 : sizeof(Probe) * (size_t)B * (size_t)gamma));
    L->tile_mass = off; off = align256(off + (topp ? 0 : sizeof(uint64_t) * (size_t)B * ntb));
    L->tile_sub = off;  off = align256(off + (topp ? 0 : sizeof(uint64_t) * (size_t)B * ntb * kSubTiles));
    L->tile_jb = off;   off = align256(off + (topp ? 0 : sizeof(int32_t) * (ntb + 1)));
    L->data_bytes = off;
    *Ct = ct;
    *Cd = cd;
    *tile = tl;
    *ntiles = nt;
    return true;
}

// ---------------------------------------------------------------------------
// Draft-side sampler
// ---------------------------------------------------------------------------
int32_t draft_chunks(int32_t B, int32_t V) {
    const int64_t want = ((int64_t)kDraftTargetWgs + (B > 0 ? B : 1) - 1) / (B > 0 ? B : 1);
    int64_t cap = (int64_t)V / kDraftMinChunk;
    if (cap < 1) cap = 1;
    int64_t C = want < cap ? want : cap;
    if (C > kDraftMaxChunks) C = kDraftMaxChunks;
    if (C < 1) C = 1;
    return (int32_t)C;
}

void draft_layout(int32_t B, int32_t V, DraftLayout *L, int32_t *C) {
    const int32_t c = draft_chunks(B, V);
    // chunk results sized by the bound that never decreases with B or V;
    // band lists whenever rows of this length can be cut at all
    const int64_t cap = (int64_t)V / kDraftMinChunk;
    const size_t nch = (size_t)chunk_total_bound(B, 1, cap, kDraftTargetWgs, kDraftMaxChunks);
    L->counter_bytes = align256(sizeof(uint32_t) * (size_t)B);
    size_t off = 0;
    L->res = off;   off = align256(off + sizeof(ChunkRes) * nch);
    L->cand = off;  off = align256(off + (cap > 1 ? sizeof(uint64_t) * nch * kCandCap : 0));
    L->desc = off;  off = align256(off + sizeof(RowDesc) * (size_t)B);
    L->data_bytes = off;
    *C = c;
}

// ---------------------------------------------------------------------------
// Vocabulary trim
// ---------------------------------------------------------------------------
namespace {
struct TrimGeom {
    int32_t R, logR, KB, S, nblocks;
};
TrimGeom trim_geom(int32_t Vt) {
    TrimGeom g;
    g.logR = 0;
    while ((((int64_t)Vt + ((int64_t)1 << g.logR) - 1) >> g.logR) > kTrimBins) ++g.logR;
    g.R = 1 << g.logR;
    g.KB = (int32_t)(((((int64_t)Vt + g.R - 1) >> g.logR) + 7) & ~(int64_t)7);    // bins per range, padded to 8
    int32_t s = kTrimTargetWgs / g.R;
    if (s < 1) s = 1;
    if (s > kTrimMaxSlices) s = kTrimMaxSlices;
    g.S = s;
    g.nblocks = (Vt + kTrimBlock - 1) / kTrimBlock;
    return g;
}
struct TrimSizes {
    size_t part, counts, hn, hm, h2, list, bd, st, total;
};
TrimSizes trim_sizes(int32_t Vt) {
    const TrimGeom g = trim_geom(Vt);
    TrimSizes z;
    // S R <= max(kTrimTargetWgs, R) and KB <= min(kTrimBins, Vt rounded up to 8): a bound
    // that never shrinks as Vt grows, so a workspace sized for one vocabulary
    // serves every smaller one
    const size_t sr = (size_t)(g.R > kTrimTargetWgs ? g.R : kTrimTargetWgs);
    const size_t kb = (size_t)(Vt < kTrimBins ? (Vt + 7) & ~7 : kTrimBins);
    z.part = align256(sizeof(uint16_t) * sr * kb);
    z.counts = align256(sizeof(uint32_t) * (size_t)Vt);
    z.hn = align256(sizeof(uint32_t) * kTrimBuckets);
    z.hm = align256(sizeof(unsigned long long) * kTrimBuckets);
    z.h2 = align256(sizeof(uint32_t) * kTrimFine);
    z.list = align256(sizeof(uint32_t) * kTrimList);
    z.bd = align256(sizeof(uint32_t) * (size_t)g.nblocks);
    z.st = align256(sizeof(TrimState));
    z.total = z.part + z.counts + z.hn + z.hm + z.h2 + z.list + 2 * z.bd + z.st;
    return z;
}
}  // namespace

// totals and arrival counters, then the per-id overflow counts
size_t trim_counter_bytes(int32_t Vt) { return 256 + align256(sizeof(uint32_t) * (size_t)Vt); }
size_t trim_data_bytes(int32_t Vt) { return trim_sizes(Vt).total; }

void trim_layout(TrimArgs &a, char *base, char *data) {
    const TrimGeom g = trim_geom(a.Vt);
    const TrimSizes z = trim_sizes(a.Vt);
    a.R = g.R;
    a.logR = g.logR;
    a.KB = g.KB;
    a.S = g.S;
    a.nblocks = g.nblocks;
    a.totals = reinterpret_cast<unsigned long long *>(base);
    a.arrive = reinterpret_cast<uint32_t *>(base + 2 * sizeof(unsigned long long));
    a.ovf = reinterpret_cast<uint32_t *>(base + 256);
    char *p = data;
    a.part = reinterpret_cast<uint32_t *>(p);
    p += z.part;
    a.counts = reinterpret_cast<uint32_t *>(p);
    p += z.counts;
    a.hist_n = reinterpret_cast<uint32_t *>(p);
    p += z.hn;
    a.hist_m = reinterpret_cast<unsigned long long *>(p);
    p += z.hm;
    a.h2 = reinterpret_cast<uint32_t *>(p);
    p += z.h2;
    a.list = reinterpret_cast<uint32_t *>(p);
    p += z.list;
    a.blockdef = reinterpret_cast<uint32_t *>(p);
    p += z.bd;
    a.blocktie = reinterpret_cast<uint32_t *>(p);
    p += z.bd;
    a.state = reinterpret_cast<TrimState *>(p);
}

// ---------------------------------------------------------------------------
// Fused lm_head
// ---------------------------------------------------------------------------
size_t lmhead_part_bytes(int64_t M, int32_t V) {
    const size_t nt = ((size_t)V + kLmTile - 1) / kLmTile;
    return align256(sizeof(uint64_t) * (size_t)M * nt);
}
size_t lmhead_data_bytes(int64_t M, int32_t V) {
    return lmhead_part_bytes(M, V) + align256(sizeof(ArgMax) * (size_t)M);
}
// GEMM column tiles (kLmGroup key tiles each), rounded up to a multiple of 8
// so that the workgroups of one column tile share an XCD
int64_t lmhead_col_tiles8(int32_t V) {
    const int64_t nt = ((int64_t)V + kLmTile - 1) / kLmTile;
    return ((nt + kLmGroup - 1) / kLmGroup + 7) / 8 * 8;
}

// ---------------------------------------------------------------------------
// Argument checks
// ---------------------------------------------------------------------------
namespace {
sv_status greedy_fit(int32_t B, int32_t R, int32_t V, size_t ws_bytes) {
    if (!workspace_fits(ws_bytes, greedy_counter_bytes(B, R, V), greedy_data_bytes(B, R, V)))
        return SV_ERR_WORKSPACE_TOO_SMALL;
    if (!grid_fits((int64_t)B * R * greedy_C(B, R, V))) return SV_ERR_TOO_LARGE;
    return SV_OK;
}
}  // namespace

sv_status check_greedy(const void *target_logits, int dtype, const int32_t *draft_tokens, int32_t B, int32_t gamma,
                       int32_t V, const int32_t *out_tokens, const int32_t *out_accept_len, const void *workspace,
                       size_t workspace_bytes, bool *launch) {
    *launch = false;
    if (!dtype_ok(dtype)) return SV_ERR_UNSUPPORTED_DTYPE;
    if (B < 0 || gamma < 0 || V < 1) return SV_ERR_INVALID_ARG;
    if (gamma > SV_MAX_GAMMA || V > SV_MAX_VOCAB) return SV_ERR_TOO_LARGE;
    if (B == 0) return SV_OK;
    if (!target_logits || !out_tokens || !out_accept_len || !workspace) return SV_ERR_INVALID_ARG;
    if (gamma > 0 && !draft_tokens) return SV_ERR_INVALID_ARG;
    if (!aligned(target_logits, esize(dtype))) return SV_ERR_INVALID_ARG;
    const sv_status f = greedy_fit(B, gamma + 1, V, workspace_bytes);
    *launch = f == SV_OK;
    return f;
}

sv_status check_tree(const void *target_logits, int dtype, const int32_t *node_tokens, const int32_t *parents,
                     int32_t B, int32_t N, int32_t V, const int32_t *out_path_nodes, const int32_t *out_tokens,
                     const int32_t *out_accept_len, const void *workspace, size_t workspace_bytes, bool *launch) {
    *launch = false;
    if (!dtype_ok(dtype)) return SV_ERR_UNSUPPORTED_DTYPE;
    if (B < 0 || N < 1 || V < 1) return SV_ERR_INVALID_ARG;
    if (N > SV_MAX_TREE_NODES || V > SV_MAX_VOCAB) return SV_ERR_TOO_LARGE;
    if (B == 0) return SV_OK;
    if (!target_logits || !node_tokens || !parents || !out_path_nodes || !out_tokens || !out_accept_len ||
        !workspace)
        return SV_ERR_INVALID_ARG;
    if (!aligned(target_logits, esize(dtype))) return SV_ERR_INVALID_ARG;
    const sv_status f = greedy_fit(B, N, V, workspace_bytes);
    *launch = f == SV_OK;
    return f;
}

sv_status check_sample(const void *target_logits, int target_dtype, const void *draft_logits, int draft_dtype,
                       const int32_t *draft_tokens, const int32_t *d2t, const float *u_accept, const float *u_sample,
                       int32_t B, int32_t gamma, int32_t Vt, int32_t Vd, float temperature, float top_p,
                       const int32_t *out_tokens, const int32_t *out_accept_len, const void *workspace,
                       size_t workspace_bytes, WorkspaceLayout *L, int32_t *Ct, int32_t *Cd, int32_t *tile,
                       int32_t *ntiles, bool *launch) {
    *launch = false;
    if (!dtype_ok(target_dtype) || !dtype_ok(draft_dtype)) return SV_ERR_UNSUPPORTED_DTYPE;
    if (B < 0 || gamma < 0 || Vt < 1 || Vd < 1) return SV_ERR_INVALID_ARG;
    if (!(temperature > 0.0f) || !isfinite(temperature)) return SV_ERR_INVALID_ARG;
    if (!(top_p > 0.0f)) return SV_ERR_INVALID_ARG;          // also rejects NaN
    if (!d2t && Vd != Vt) return SV_ERR_INVALID_ARG;
    if (d2t && Vd > Vt) return SV_ERR_INVALID_ARG;            // an injective map needs Vd <= Vt
    if (gamma > SV_MAX_GAMMA || Vt > SV_MAX_VOCAB || Vd > SV_MAX_VOCAB) return SV_ERR_TOO_LARGE;
    if (B == 0) return SV_OK;
    if (!target_logits || !u_sample || !out_tokens || !out_accept_len || !workspace) return SV_ERR_INVALID_ARG;
    if (gamma > 0 && (!draft_logits || !draft_tokens || !u_accept)) return SV_ERR_INVALID_ARG;
    if (!aligned(target_logits, esize(target_dtype))) return SV_ERR_INVALID_ARG;
    if (gamma > 0 && !aligned(draft_logits, esize(draft_dtype))) return SV_ERR_INVALID_ARG;
    const bool topp = top_p < 1.0f;
    sample_layout(B, gamma, Vt, Vd, (int32_t)esize(target_dtype), (int32_t)esize(draft_dtype), topp, L, Ct, Cd, tile,
                  ntiles);
    if (!workspace_fits(workspace_bytes, L->counter_bytes, L->data_bytes)) return SV_ERR_WORKSPACE_TOO_SMALL;
    const int64_t NR = 2 * (int64_t)gamma + 1;
    if (!grid_fits((int64_t)B * (topp ? NR : (1 + (int64_t)(gamma + 1) * *Ct + (int64_t)gamma * *Cd))) ||
        !grid_fits((int64_t)B * *ntiles))
        return SV_ERR_TOO_LARGE;
    *launch = true;
    return SV_OK;
}

sv_status check_draft(const void *logits, int dtype, const float *u, int32_t B, int32_t V, float temperature,
                      float top_p, const int32_t *out_tokens, const void *workspace, size_t workspace_bytes,
                      DraftLayout *L, int32_t *C, bool *launch) {
    *launch = false;
    if (!dtype_ok(dtype)) return SV_ERR_UNSUPPORTED_DTYPE;
    if (B < 0 || V < 1) return SV_ERR_INVALID_ARG;
    if (!(temperature > 0.0f) || !isfinite(temperature)) return SV_ERR_INVALID_ARG;
    if (!(top_p > 0.0f)) return SV_ERR_INVALID_ARG;
    if (V > SV_MAX_VOCAB) return SV_ERR_TOO_LARGE;
    if (B == 0) return SV_OK;
    if (!logits || !u || !out_tokens || !workspace) return SV_ERR_INVALID_ARG;
    if (!aligned(logits, esize(dtype))) return SV_ERR_INVALID_ARG;
    draft_layout(B, V, L, C);
    if (!workspace_fits(workspace_bytes, L->counter_bytes, L->data_bytes)) return SV_ERR_WORKSPACE_TOO_SMALL;
    if (!grid_fits((int64_t)B * *C)) return SV_ERR_TOO_LARGE;
    *launch = true;
    return SV_OK;
}

sv_status check_count(const int32_t *accept_len, int32_t B, int32_t gamma, const uint64_t *counters, bool *launch) {
    *launch = false;
    if (B < 0 || gamma < 0) return SV_ERR_INVALID_ARG;
    if (gamma > SV_MAX_GAMMA) return SV_ERR_TOO_LARGE;
    if (B == 0) return SV_OK;
    if (!accept_len || !counters) return SV_ERR_INVALID_ARG;
    if (!aligned(counters, sizeof(uint64_t))) return SV_ERR_INVALID_ARG;
    *launch = true;
    return SV_OK;
}

sv_status check_fanout(const int32_t *out_tokens, const int32_t *accept_len, const int32_t *cand,
                       const int32_t *branch_drafts, int32_t B, int32_t gamma, int32_t f, int32_t L,
                       const int32_t *out_branch, const int32_t *out_next, const uint64_t *counters, bool *launch) {
    *launch = false;
    if (B < 0 || gamma < 0 || f < 1 || L < 0) return SV_ERR_INVALID_ARG;
    if (gamma > SV_MAX_GAMMA || f > SV_MAX_FANOUT || L > SV_MAX_BRANCH_DRAFTS) return SV_ERR_TOO_LARGE;
    if (B == 0) return SV_OK;
    if (!out_tokens || !accept_len || !cand || !out_branch) return SV_ERR_INVALID_ARG;
    if (out_next && L > 0 && !branch_drafts) return SV_ERR_INVALID_ARG;
    if (counters && !aligned(counters, sizeof(uint64_t))) return SV_ERR_INVALID_ARG;
    if (!grid_fits(((int64_t)B + 3) / 4)) return SV_ERR_TOO_LARGE;
    *launch = true;
    return SV_OK;
}

sv_status check_trim(const int32_t *tokens, int64_t N, int32_t Vt, float P, const int32_t *out_d2t,
                     const int32_t *out_vd, const int64_t *out_info, const void *workspace, size_t workspace_bytes,
                     bool *launch) {
    *launch = false;
    if (N < 0 || Vt < 1 || !(P > 0.0f)) return SV_ERR_INVALID_ARG;
    if (Vt > SV_MAX_VOCAB || N > (int64_t)INT32_MAX) return SV_ERR_TOO_LARGE;
    if ((N > 0 && !tokens) || !out_d2t || !out_vd || !workspace) return SV_ERR_INVALID_ARG;
    if (out_info && !aligned(out_info, sizeof(int64_t))) return SV_ERR_INVALID_ARG;
    if (!workspace_fits(workspace_bytes, trim_counter_bytes(Vt), trim_data_bytes(Vt))) return SV_ERR_WORKSPACE_TOO_SMALL;
    *launch = true;
    return SV_OK;
}

sv_status check_lmhead(const void *hidden, const void *W, const int32_t *tokens, const int32_t *parents, bool tree,
                       int32_t B, int32_t R, int32_t d, int32_t V, const int32_t *out_path_nodes,
                       const int32_t *out_tokens, const int32_t *out_accept_len, const void *workspace,
                       size_t workspace_bytes, bool *launch) {
    *launch = false;
    if (tree) {
        if (R > SV_MAX_TREE_NODES) return SV_ERR_TOO_LARGE;
    } else {
        if (R < 1) return SV_ERR_INVALID_ARG;                 // R = gamma + 1
        if (R - 1 > SV_MAX_GAMMA) return SV_ERR_TOO_LARGE;
    }
    if (B < 0 || R < 1 || d < 8 || V < 1) return SV_ERR_INVALID_ARG;
    if (d % 8 != 0) return SV_ERR_INVALID_ARG;
    if (V > SV_MAX_VOCAB) return SV_ERR_TOO_LARGE;
    if (B == 0) return SV_OK;
    if (!hidden || !W || !aligned(hidden, 16) || !aligned(W, 16)) return SV_ERR_INVALID_ARG;
    if (tree) {
        if (!tokens || !parents || !out_path_nodes || !out_tokens || !out_accept_len || !workspace)
            return SV_ERR_INVALID_ARG;
    } else if (!out_tokens || !out_accept_len || !workspace || (R > 1 && !tokens)) {
        return SV_ERR_INVALID_ARG;
    }
    const int64_t M = (int64_t)B * R;
    if (M > INT32_MAX) return SV_ERR_TOO_LARGE;
    if (!workspace_fits(workspace_bytes, 256, lmhead_data_bytes(M, V))) return SV_ERR_WORKSPACE_TOO_SMALL;
    const int64_t mtiles = (M + kLmTile - 1) / kLmTile;
    if (!grid_fits(mtiles * lmhead_col_tiles8(V))) return SV_ERR_TOO_LARGE;
    *launch = true;
    return SV_OK;
}

}  // namespace sv

using namespace sv;

extern "C" {

const char *spec_verify_strerror(sv_status s) {
    switch (s) {
        case SV_OK: return "ok";
        case SV_ERR_INVALID_ARG: return "invalid argument";
        case SV_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
        case SV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SV_ERR_HIP: return "HIP launch error";
        case SV_ERR_TOO_LARGE: return "size beyond library limits";
    }
    return "unknown status";
}

size_t sv_workspace_bytes_greedy(int32_t B, int32_t gamma, int32_t V) {
    if (B < 0 || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB) return 0;
    return greedy_ws(B, gamma + 1, V);
}

size_t sv_workspace_bytes_tree(int32_t B, int32_t N, int32_t V) {
    if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB) return 0;
    return greedy_ws(B, N, V);
}

size_t sv_workspace_bytes_sample(int32_t B, int32_t gamma, int32_t Vt, int32_t Vd, float top_p) {
    if (B < 0 || gamma < 0 || gamma > SV_MAX_GAMMA || Vt < 1 || Vd < 1 || Vt > SV_MAX_VOCAB ||
        Vd > SV_MAX_VOCAB || !(top_p > 0.0f))
        return 0;
    WorkspaceLayout L;
    int32_t ct, cd, tl, nt;
    sample_layout(B, gamma, Vt, Vd, 4, 4, top_p < 1.0f, &L, &ct, &cd, &tl, &nt);
    return workspace_need(L.counter_bytes, L.data_bytes);
}

size_t sv_workspace_bytes_draft(int32_t B, int32_t V) {
    if (B < 0 || V < 1 || V > SV_MAX_VOCAB) return 0;
    DraftLayout L;
    int32_t C;
    draft_layout(B, V, &L, &C);
    return workspace_need(L.counter_bytes, L.data_bytes);
}

size_t sv_workspace_bytes_vocab_trim(int32_t Vt) {
    if (Vt < 1 || Vt > SV_MAX_VOCAB) return 0;
    return workspace_need(trim_counter_bytes(Vt), trim_data_bytes(Vt));
}

size_t sv_workspace_bytes_lmhead(int32_t M, int32_t V) {
    if (M < 0 || V < 1 || V > SV_MAX_VOCAB) return 0;
    return workspace_need(256, lmhead_data_bytes(M, V));
}

}  // extern "C"
